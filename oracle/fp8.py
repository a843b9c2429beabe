"""Per-token dynamic FP8 E4M3 activation quantisation (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

robotworld.top SparkDiffusion write-up, section 2.3: projections run W8A8
in FP8 E4M3; activations get a dynamic scale per token at run time, and the
scale and the type conversion happen in one pass over memory.

Readings where the page is silent:
  * the format is the OCP "E4M3FN" one the NVIDIA targets use: 1 sign,
    4 exponent (bias 7) and 3 mantissa bits, no infinities, NaN = S.1111.111,
    largest finite 448, subnormals m * 2^-9;
  * per row m: amax = max_k |x_mk| (floored at 1e-12 so a zero row stays
    finite); the stored scale is the dequantisation multiplier
    s = fp32(amax / 448) (one correctly rounded float32 division);
  * the code of x is E4M3(x / s): the quotient of the element by the stored
    scale, rounded to nearest with ties to the even code, saturating to
    +-448. The quotient is formed in float64. That rounding never decides a
    code: x has 8 significant bits and s 24, so a quotient that is not
    exactly an E4M3 midpoint (5 significant bits) lies at least 2^-29 of its
    size away from it, far beyond float64's 2^-53.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
AMAX_FLOOR = np.float32(1e-12)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN code (0..255) -> float64 value (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# The 127 non-negative finite values, indexed by their code (monotone).
_POS_VALUES = e4m3_decode(np.arange(127))


def e4m3_encode(v) -> np.ndarray:
    """float64 -> E4M3FN code: round to nearest, ties to the even code
    (last mantissa bit 0), |v| > 448 saturates to +-448, NaN -> 0x7F.
    Negative zero encodes as 0x80.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    a_c = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a_c, side="left")  # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a_c
    d_lo = a_c - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a_c == _POS_VALUES[hi], hi, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def quant_fp8_per_token(x_bits):
    """x [M, K] bf16 bits -> (codes uint8 [M, K], scales float32 [M]).

    amax per row (exact), s = fp32(max(amax, 1e-12) / 448), codes =
    E4M3(x / s) with the quotient in float64.
    """
    xb = np.asarray(x_bits, dtype=np.uint16)
    x = (xb.astype(np.uint32) << 16).view(np.float32)  # exact widening
    amax = np.max(np.abs(x), axis=1)
    amax = np.maximum(amax, AMAX_FLOOR).astype(np.float32)
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)     # IEEE fp32 division
    v = x.astype(np.float64) / scales.astype(np.float64)[:, None]
    codes = e4m3_encode(v)
    return codes, scales
