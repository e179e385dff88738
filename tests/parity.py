"""Comparison metrics shared by the GPU parity tests."""

import numpy as np


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    return float(a @ b / (na * nb))


def max_rel(gpu, ref):
    """max_i |gpu_i - ref_i| / max_i |ref_i| (normalised by the tensor's max,
    since the element-wise ratio is undefined where ref is zero)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return float(np.max(np.abs(gpu)))
    return float(np.max(np.abs(gpu - ref)) / scale)


def bf16_round(a):
    """Round-to-nearest-even to bfloat16, returned as float32."""
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)
