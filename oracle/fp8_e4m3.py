"""The 8-bit floating-point format of an FP8 KV cache, decoded and encoded
from its definition, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P2] "量化压缩KV Cache的INT8与FP8方案" names an FP8 cache format that needs
hardware support and writes it "E4M1", which cannot be right for an 8-bit
float with a sign bit (1 + 4 + 1 = 6 bits).  The reading taken here is the
OCP FP8 E4M3 format, the one both current hardware generations the page has in
mind and the target GPU convert natively:

* bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the
  mantissa field m;
* e = 0 is subnormal: value = m / 8 * 2**-6 (so the smallest step is 2**-9);
* otherwise value = (1 + m / 8) * 2**(e - 7);
* there are no infinities: e = 15 with m = 7 (codes 0x7F and 0xFF) is NaN, so
  the largest finite magnitude is 1.75 * 2**8 = 448 (code 0x7E).

Encoding (the cache write) rounds to the nearest representable value, ties
to the code with an even mantissa, and saturates: every magnitude above 448,
infinities included, becomes +-448 (a saturating encoder is this library's
reading: the page says nothing about overflow).  NaN encodes as 0x7F.
Pins: tests/test_oracle_fp8.py (all 256 codes against torch's float8_e4m3fn,
closed forms, the encoder against torch's rounding, and round trips).
"""
import numpy as np

MAX_FINITE = 448.0


def decode(codes):
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    magnitude = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    magnitude = np.where((e == 15) & (c & 0x7 == 7), np.nan, magnitude)
    return sign * magnitude


# The 127 non-negative finite values, increasing with the code 0x00 .. 0x7E.
_GRID = decode(np.arange(0x7F))


def encode(x):
    """float values -> uint8 codes: nearest value, ties to even mantissa,
    magnitudes above 448 saturate, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_a, flat_out, flat_x = a.reshape(-1), out.reshape(-1), x.reshape(-1)
    for i in range(flat_a.size):
        v = flat_a[i]
        if np.isnan(v):
            flat_out[i] = 0x7F
            continue
        if v >= MAX_FINITE:
            code = 0x7E
        else:
            hi = int(np.searchsorted(_GRID, v, side="left"))  # first grid value >= v
            if _GRID[hi] == v:
                code = hi
            else:
                lo = hi - 1
                dlo, dhi = v - _GRID[lo], _GRID[hi] - v
                if dlo < dhi:
                    code = lo
                elif dhi < dlo:
                    code = hi
                else:
                    code = lo if lo % 2 == 0 else hi   # the even mantissa
        flat_out[i] = code | (0x80 if np.signbit(flat_x[i]) else 0)
    return out
