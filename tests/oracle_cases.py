"""Tiny fixed problems shared by the oracle pin tests (CPU only)."""
import numpy as np


def tiny_problem(n, d, v, k, seed, masked=(), w_scale=0.7, logit_scale=2.0, unmatched=False):
    """Exact float64 values that are also exact float32 values.  unmatched:
    plant ids outside [0, v) -- v itself, -1, 2^24 + 1 (an in-vocabulary id
    in its low 24 bits) and INT_MIN -- in rows 0..2 (needs n >= 3, k >= 4)."""
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    W = (w_scale * rng.standard_normal((v, d))).astype(np.float32).astype(np.float64)
    ids = np.stack([rng.permutation(v)[:k] for _ in range(n)]).astype(np.int64)
    if unmatched:
        ids[0, 1] = v
        ids[1, 0] = -1
        ids[1, 3] = (1 << 24) + 1
        ids[2, 2] = -(1 << 31)
    a = (logit_scale * rng.standard_normal((n, k))).astype(np.float32).astype(np.float64)
    a = -np.sort(-a, axis=1)
    mask = None
    if masked:
        mask = np.ones(n, dtype=np.uint8)
        mask[list(masked)] = 0
    return H, W, ids, a, mask


# (name, n, d, v, k, seed, masked rows); a name ending in "-unmatched" plants
# ids outside the vocabulary (tiny_problem's unmatched)
TINY = [
    ("n3d4v7k3-masked", 3, 4, 7, 3, 11, (1,)),
    ("n2d3v5k1", 2, 3, 5, 1, 12, ()),
    ("n4d5v11k3", 4, 5, 11, 3, 13, ()),
    ("n3d2v9k9-fullK", 3, 2, 9, 9, 14, (2,)),
    ("n4d3v8k4-unmatched", 4, 3, 8, 4, 15, (3,)),
]


def case_problem(spec, seed_offset=0, **kw):
    """tiny_problem for a TINY entry."""
    name, n, d, v, k, seed, masked = spec
    return tiny_problem(n, d, v, k, seed + seed_offset, masked, unmatched=name.endswith("-unmatched"), **kw)
