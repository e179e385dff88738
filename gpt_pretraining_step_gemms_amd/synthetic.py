"""Seeded synthetic inputs shared by the HIP path's tests and the oracle.

This module holds no arithmetic of the model or of the optimizer: only token
ids and initial weights drawn from numpy's PCG64 generator.

* Token rows: T+1 ids per row; inputs are ids[:, :-1], targets ids[:, 1:]
  (next-token prediction).  Ids are i.i.d. uniform over the vocabulary, or
  truncated Zipf(s) with P(id = k) proportional to (k + 1)^-s for
  k = 0..V-1 (rank = id, no permutation).
* Weights: i.i.d. N(0, std^2), one generator per (seed, parameter name), so
  the draw of a tensor does not depend on the order tensors are made in.
"""

import zlib

import numpy as np


def _rng(*keys):
    return np.random.Generator(np.random.PCG64(list(keys)))


def zipf_cdf(V, s):
    w = (np.arange(1, V + 1, dtype=np.float64)) ** (-float(s))
    c = np.cumsum(w)
    return c / c[-1]


def token_rows(seed, B, T, V, dist="zipf", s=1.1):
    """Returns (tokens, targets), int32 arrays [B, T]."""
    rng = _rng(int(seed), 7)
    if dist == "uniform":
        ids = rng.integers(0, V, size=(B, T + 1), dtype=np.int64)
    elif dist == "zipf":
        u = rng.random(size=(B, T + 1))
        ids = np.searchsorted(zipf_cdf(V, s), u, side="right")
        ids = np.minimum(ids, V - 1)
    else:
        raise ValueError(dist)
    ids = ids.astype(np.int32)
    return np.ascontiguousarray(ids[:, :-1]), np.ascontiguousarray(ids[:, 1:])


def normal_tensor(seed, name, shape, std):
    """float32 tensor of i.i.d. N(0, std^2) values for parameter ``name``."""
    rng = _rng(int(seed), zlib.crc32(name.encode()))
    return (rng.standard_normal(size=shape) * std).astype(np.float32)


def normal_params(seed, shapes, std):
    """name -> float32 array for every (name, shape) in ``shapes``."""
    return {n: normal_tensor(seed, n, s, std) for n, s in shapes.items()}


def normal_matrix(seed, rows, cols, std=1.0, dtype=np.float32):
    rng = _rng(int(seed), 11)
    return (rng.standard_normal(size=(rows, cols)) * std).astype(dtype)
