"""Pins of the oracle's FP8 E4M3 codec (CPU): against torch's float8_e4m3fn,
closed forms of the format, round trips, and planted mistakes."""
import types

import numpy as np
import pytest
import torch

import oracle.fp8_e4m3 as f8

CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_decode_matches_torch(mod):
    assert np.array_equal(mod.decode(CODES), _torch_decode(CODES), equal_nan=True)


def pin_closed_forms(mod):
    d = lambda c: float(mod.decode(np.array([c]))[0])  # noqa: E731
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9  # subnormals
    assert d(0x08) == 2.0 ** -6                               # smallest normal
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x3C) == 1.5
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x00) == 0.0 and np.signbit(d(0x80))


def pin_encode_matches_torch(mod):
    """Within range the encoder is round-to-nearest-even onto the grid, as
    torch's conversion is; values, exact midpoints (ties) and both signs."""
    rng = np.random.default_rng(3)
    grid = f8.decode(np.arange(0x7F))
    mids = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([rng.standard_normal(4000) * rng.choice([1e-3, 0.05, 1, 30, 300], 4000),
                        mids, -mids, grid, -grid, [0.0, -0.0]]).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(mod.encode(x), _torch_encode(x))


def pin_saturation_and_nan(mod):
    e = lambda v: int(mod.encode(np.array([v]))[0])  # noqa: E731
    assert e(448.0) == 0x7E and e(449.0) == 0x7E and e(1e30) == 0x7E and e(np.inf) == 0x7E
    assert e(-500.0) == 0xFE and e(-np.inf) == 0xFE
    assert e(np.nan) == 0x7F
    assert e(-1e-9) == 0x80 and e(1e-9) == 0x00


def pin_round_trip(mod):
    finite = CODES[~np.isnan(f8.decode(CODES))]
    assert np.array_equal(mod.encode(mod.decode(finite)), finite)


PINS = [pin_decode_matches_torch, pin_closed_forms, pin_encode_matches_torch,
        pin_saturation_and_nan, pin_round_trip]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_pins(pin):
    pin(f8)


MUTATIONS = {
    "bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "mantissa_over_16": ("(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    "subnormal_exponent": ("m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    "no_nan_code": ("np.where((e == 15) & (c & 0x7 == 7), np.nan, magnitude)", "magnitude"),
    "ties_away": ("code = lo if lo % 2 == 0 else hi", "code = hi"),
    "ties_down": ("code = lo if lo % 2 == 0 else hi", "code = lo"),
    "no_saturation": ("        if v >= MAX_FINITE:\n            code = 0x7E\n        else:\n", "        if True:\n"),
    "sign_dropped": ("flat_out[i] = code | (0x80 if np.signbit(flat_x[i]) else 0)", "flat_out[i] = code"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_fp8_pins_catch_mutation(name):
    old, new = MUTATIONS[name]
    src = open(f8.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"fp8_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {name}"
