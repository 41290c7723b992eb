"""The decode and cache-write oracle against its pins (CPU only)."""
import pytest

import oracle.paged_attention as pa
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_DECODE_PINS, ids=lambda f: f.__name__)
def test_decode_pin(pin):
    pin(pa)


@pytest.mark.parametrize("pin", oracle_pins.ALL_CACHE_WRITE_PINS, ids=lambda f: f.__name__)
def test_cache_write_pin(pin):
    pin(pa)


def test_table_past_pool_raises():
    import numpy as np
    kc = np.zeros((2, 16, 1, 4), np.float32)
    with pytest.raises(IndexError):
        pa.paged_decode(np.zeros((1, 1, 4), np.float32), "f32", kc, kc, "f32",
                        np.array([[0, 5]], np.int32), [20], 16, 1.0)
    with pytest.raises(IndexError):
        pa.paged_decode(np.zeros((1, 1, 4), np.float32), "f32", kc, kc, "f32",
                        np.array([[0]], np.int32), [20], 16, 1.0)
