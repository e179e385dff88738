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

Gradients (the backward products, when those run in fp8) use e5m2 of the
same specification: 5 exponent bits with bias 15, 2 mantissa bits, largest
finite value 57344 (exponent 31 holds infinities and NaNs).  Reading: the
page names only tensorwise scaling, and e5m2 for gradients is the usual
companion of e4m3 in fp8 training (a wider range for gradient values); the
scale is s = 57344 / max|x|, with the same rounding, saturation and NaN rules
(NaN -> 0x7F, a NaN of that format).

The encoder here works from the table of all representable values: a plain
nearest-value search, not the bit manipulation of the HIP kernel.
"""

E4M3, E5M2 = "e4m3", "e5m2"
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}

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
    return _encode(x, _POS, 0x7E, 0x7F)


def e4m3_decode(codes):
    return _TABLE[np.asarray(codes, np.uint8)]


def bf16_round(x):
    """Round to bfloat16 (nearest, ties to even), returned as float64: the
    fp8 operands of the forward products are quantised from their bf16 copies
    (the stored activations and weight copies of the bf16 configuration)."""
    u = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def e5m2_decode_table():
    """float64 value of every e5m2 code 0..255 (inf for the two infinity
    codes, NaN for the six NaN codes)."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 2) & 0x1F, c & 3
        if e == 0x1F:
            vals[c] = sign * np.inf if m == 0 else np.nan
        elif e == 0:
            vals[c] = sign * (m / 4.0) * 2.0 ** -14
        else:
            vals[c] = sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return vals


_TABLE5 = e5m2_decode_table()
_POS5 = _TABLE5[:0x7C]               # codes 0x00 .. 0x7B: 0 .. 57344, increasing


def _encode(x, pos, top, nan_code):
    x = np.asarray(x, np.float64)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), pos[top])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, top)
    lo = np.clip(hi - 1, 0, top)
    d_lo, d_hi = a - pos[lo], pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code)
    return np.where(nan, nan_code, code).astype(np.uint8)


def e5m2_encode(x):
    """Codes of float values x: nearest of the 124 non-negative finite e5m2
    values to |x| (saturating at 57344), ties to the even code, sign from x;
    NaN -> 0x7F."""
    return _encode(x, _POS5, 0x7B, 0x7F)


def e5m2_decode(codes):
    return _TABLE5[np.asarray(codes, np.uint8)]


def encode(x, fmt):
    return e4m3_encode(x) if fmt == E4M3 else e5m2_encode(x)


def decode(codes, fmt):
    return e4m3_decode(codes) if fmt == E4M3 else e5m2_decode(codes)


def quantize_tensorwise(x, fmt=E4M3):
    """(codes, amax, scale) of a tensor: scale = FMT_MAX / amax in fp32
    (448 for e4m3, 57344 for e5m2), codes of x * scale evaluated in fp32."""
    x32 = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if np.isnan(amax):
        scale = np.float32(np.nan)
    else:
        scale = np.float32(FMT_MAX[fmt]) / amax if amax > 0 else np.float32(1.0)
    return encode((x32 * scale).astype(np.float32), fmt), float(amax), float(scale)


def dequantized(x, fmt=E4M3):
    """The values an fp8 product sees for tensor x: decode(codes) / scale."""
    codes, _, scale = quantize_tensorwise(x, fmt)
    return decode(codes, fmt) / scale


def fp8_matmul(a_codes, b_codes, alpha, a_fmt=E4M3, b_fmt=E4M3):
    """alpha * A B^T of two code matrices [M, K], [N, K], in fp64."""
    return alpha * (decode(a_codes, a_fmt) @ decode(b_codes, b_fmt).T)
