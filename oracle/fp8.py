"""OCP fp8 e4m3 encoding and tensorwise scaling, in numpy — TEST INFRASTRUCTURE
ONLY (see the package docstring).

[APIDOG] "3. Manajemen Presisi (nanochat/common.py)": later runs train most
linear layers in FP8 with tensorwise scaling.  Readings where the page is
silent: the format is e4m3 of the OCP 8-bit floating point specification
(sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 15 with mantissa
7 is NaN, so the largest finite value is 448; no infinities); the tensorwise
scale is s = 448 / max|x| (1 when x is all zero), computed in fp32, and a
value x is stored as e4m3(x * s), the product taken in fp32, rounded to the
nearest representable value with ties to the even code, saturating at 448.
A NaN is stored as the code 0x7F (the format's NaN, sign bit clear), and a
NaN anywhere in a tensor makes its amax and scale NaN, so every code of that
tensor is 0x7F: the error reaches the product instead of becoming a finite
value.

The encoder here works from the table of all representable values: a plain
nearest-value search, not the bit manipulation of the HIP kernel.
"""

import numpy as np


def e4m3_decode_table():
    """float64 value of every code 0..255 (NaN for the two NaN codes)."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
_POS = _TABLE[:0x7F]                 # codes 0x00 .. 0x7E: 0 .. 448, increasing


def e4m3_encode(x):
    """Codes (uint8) of float values x: nearest of the 127 non-negative finite
    values to |x| (|x| above 448 saturates), ties to the even code, sign bit
    from x; NaN -> 0x7F."""
    x = np.asarray(x, np.float64)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), 448.0)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code)
    return np.where(nan, 0x7F, code).astype(np.uint8)


def e4m3_decode(codes):
    return _TABLE[np.asarray(codes, np.uint8)]


def bf16_round(x):
    """Round to bfloat16 (nearest, ties to even), returned as float64: the
    fp8 operands of the forward products are quantised from their bf16 copies
    (the stored activations and weight copies of the bf16 configuration)."""
    u = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def quantize_tensorwise(x):
    """(codes, amax, scale) of a tensor: scale = 448 / amax in fp32, codes of
    x * scale evaluated in fp32."""
    x32 = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if np.isnan(amax):
        scale = np.float32(np.nan)
    else:
        scale = np.float32(448.0) / amax if amax > 0 else np.float32(1.0)
    return e4m3_encode((x32 * scale).astype(np.float32)), float(amax), float(scale)


def fp8_matmul(a_codes, b_codes, alpha):
    """alpha * A B^T of two code matrices [M, K], [N, K], in fp64."""
    return alpha * (e4m3_decode(a_codes) @ e4m3_decode(b_codes).T)
