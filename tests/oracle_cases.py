"""Tiny fixed problems shared by the oracle pin tests (CPU only)."""
import numpy as np


def tiny_problem(n, d, v, k, seed, masked=(), w_scale=0.7, logit_scale=2.0):
    """Exact float64 values that are also exact float32 values."""
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    W = (w_scale * rng.standard_normal((v, d))).astype(np.float32).astype(np.float64)
    ids = np.stack([rng.permutation(v)[:k] for _ in range(n)]).astype(np.int64)
    a = (logit_scale * rng.standard_normal((n, k))).astype(np.float32).astype(np.float64)
    a = -np.sort(-a, axis=1)
    mask = None
    if masked:
        mask = np.ones(n, dtype=np.uint8)
        mask[list(masked)] = 0
    return H, W, ids, a, mask


# (name, n, d, v, k, seed, masked rows)
TINY = [
    ("n3d4v7k3-masked", 3, 4, 7, 3, 11, (1,)),
    ("n2d3v5k1", 2, 3, 5, 1, 12, ()),
    ("n4d5v11k3", 4, 5, 11, 3, 13, ()),
    ("n3d2v9k9-fullK", 3, 2, 9, 9, 14, (2,)),
]
