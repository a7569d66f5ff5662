"""Number formats used by the codec (oracle; test infrastructure only).

The pages name two formats: FP16 tensors and an FP8 per-group scale produced by
a per-tensor FP16-to-FP8 scale factor (Ecco review, Fig. 4 caption: "normalized
using a per-tensor FP16-to-FP8 scale factor, with the resulting normalized FP8
value serving as the group scale factor"; "Core claim": "normalized by a
per-group FP8 scale factor").  They do not say which FP8.  Reading used here:
OCP FP8 E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, 0x7F/0xFF are NaN, largest finite 448, smallest subnormal 2**-9),
with saturation to +-448 and round-to-nearest-even, never producing NaN.

Everything here is written from the format definitions, one value at a time in
float64 arithmetic that is exact for these sizes.
"""

import numpy as np

FP8_MAX = 448.0
FP8_MIN_NORMAL_EXP = -6      # smallest normal: 2**-6
FP8_SUBNORMAL_STEP = 2.0 ** -9


def _round_half_even(v):
    """Round float64 array to the nearest integer, ties to even (np.rint)."""
    return np.rint(v)


def fp8_encode(v):
    """float32 array -> uint8 array of E4M3FN codes (saturating, RNE).

    Steps: take the sign; clamp the magnitude to 448; below 2**-6 quantise to
    multiples of 2**-9 (subnormals; a result of 8 steps is the smallest normal,
    whose code is also 8); otherwise split |v| = m * 2**e with m in [1, 2),
    round (m - 1) * 8 to an integer q, carry q == 8 into the exponent, and
    emit ((e + 7) << 3) | q.  NaN input (outside the codec's precondition of
    finite tensors) maps to 0x7F.
    """
    v = np.asarray(v, dtype=np.float32)
    out = np.zeros(v.shape, dtype=np.uint8)
    vd = v.astype(np.float64)
    nan = np.isnan(vd)
    sign = np.signbit(vd)
    mag = np.minimum(np.abs(np.where(nan, 0.0, vd)), FP8_MAX)

    sub = mag < 2.0 ** FP8_MIN_NORMAL_EXP
    q_sub = _round_half_even(mag / FP8_SUBNORMAL_STEP)       # 0..8, exact scaling
    code_sub = q_sub.astype(np.int64)

    m, e = np.frexp(np.where(sub, 1.0, mag))                 # mag = m * 2**e, m in [0.5, 1)
    m = m * 2.0
    e = e - 1                                                 # mag = m * 2**e, m in [1, 2)
    q = _round_half_even((m - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    q = np.where(carry, 0, q)
    e = np.where(carry, e + 1, e)
    code_norm = ((e + 7) << 3) | q

    code = np.where(sub, code_sub, code_norm)
    code = code | np.where(sign, 0x80, 0)
    code = np.where(nan, 0x7F, code)
    out[...] = code.astype(np.uint8)
    return out


def fp8_decode(b):
    """uint8 array of E4M3FN codes -> exact float32 values (0x7F/0xFF -> NaN)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * FP8_SUBNORMAL_STEP, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    val = np.where(s == 1, -mag, mag)
    return val.astype(np.float32)


def fp16_rne(v):
    """float32 array -> float16 array, round to nearest even (IEEE cast)."""
    return np.asarray(v, dtype=np.float32).astype(np.float16)


def fp16_bits(h):
    return np.asarray(h, dtype=np.float16).view(np.uint16)


def f32(v):
    return np.float32(v)
