"""OCP E4M3 (``float8_e4m3fn``) decode and quantize, the plain way (TEST INFRASTRUCTURE).

The pages store the KV cache as ``torch.float8_e4m3fn`` (prhub digest of vLLM
PR #48666, Key code, the ``flash_attn_varlen_func`` excerpt).  Q is quantized
to that format with a static per-tensor scale before the native FP8 forward
(vLLM PR #63139, Overview: the sliding-window layers quantize Q to FP8 the
same way the FA3 path already did).  The pages do not
spell out the rounding.  The reading adopted here is IEEE fp32 division by the
descale, then round-to-nearest-even with saturation at +-448.  A NaN keeps its
sign as code 0x7F | sign.  This module implements exactly that rule and nothing
faster.

The sign of every code is the sign IEEE division gives the quotient: sign(x)
XOR sign(descale).  That includes a NaN quotient, so 0 / 0 (an all-zero tensor
gets descale amax / 448 = 0) gives 0x7F for +0 and 0xFF for -0.  (IEEE leaves
the sign of a NaN that an invalid operation creates to the platform; numpy on
x86 makes it negative.  The rule here fixes it to the sign of the operands.)
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of one E4M3 code: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.

    Exponent field 0 is subnormal (m/8 * 2^-6).  Exponent 15 with mantissa 7 is
    NaN.  The format has no infinity, so its largest finite value is 0x7E = 448."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
E4M3_TABLE.setflags(write=False)
# the 127 finite non-negative values, codes 0x00..0x7E, strictly increasing
_POS = E4M3_TABLE[:127].copy()


def dequantize_e4m3(codes, descale=1.0) -> np.ndarray:
    """fp64 value of each code times the fp32 descale (table lookup, then one exact fp64 product)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return E4M3_TABLE[codes] * float(np.float32(descale))


def quantize_e4m3(x, descale=1.0) -> np.ndarray:
    """Codes for x / descale, computed in fp32 and rounded to the nearest E4M3 value.

    Steps:
      1. y = float32(x) / float32(descale), one IEEE binary32 division (RNE).
      2. NaN gives 0x7F with the quotient's sign.
      3. |y| >= 448 (including inf) saturates to 0x7E with y's sign.
      4. Otherwise pick the E4M3 magnitude nearest to |y|, comparing in fp64.
         Both operands are exact there, so the comparison is exact.  A tie goes
         to the even code, i.e. the even mantissa.  -0 gives 0x80.
    The quotient's sign is sign(x) XOR sign(descale), the IEEE rule for
    division, taken for NaN quotients too (see the module docstring).
    """
    x32 = np.asarray(x, dtype=np.float32)
    d32 = np.float32(descale)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = (x32 / d32).astype(np.float32)
    a = np.abs(y.astype(np.float64))
    sign = np.where(np.signbit(x32) ^ np.signbit(d32), 0x80, 0x00).astype(np.uint8)
    nan = np.isnan(a)
    a_f = np.where(nan, 0.0, a)
    hi = np.clip(np.searchsorted(_POS, a_f, side="left"), 0, 126)   # _POS[hi] >= a (or 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a_f - _POS[lo]
    d_hi = _POS[hi] - a_f
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a_f >= E4M3_MAX, 0x7E, mag)
    mag = np.where(nan, 0x7F, mag).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def descale_from_amax(x) -> np.float32:
    """Per-tensor descale: float32(amax|x|) / float32(448), one fp32 division."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32))))
    return np.float32(amax / np.float32(E4M3_MAX))
