"""fp64 CPU oracle of the teacher top-K cache (test infrastructure).

TEST INFRASTRUCTURE ONLY.  This module may be imported, called or executed by
``tests/`` -- nothing else.  The HIP library and its Python binding never
import it, and it imports nothing from them.

What it computes
----------------
The offline cache the loss consumes is made once from the teacher: per
position, the 100 most probable tokens -- their ids and their logits -- are
kept, so the teacher never has to be resident during student training
(agentlenshq.com page "LLMのための効率的な知識蒸留…", section
"1. Top-K Logit Cachingによるオフライン蒸留"; aivibenews.ru page "Дистилляция
LLM на одной GPU…", section "Два приёма"; aihot.vn page "Tối ưu hóa chi phí
chưng cất tri thức…", section "Hai thay đổi hệ thống").

Softmax is strictly increasing, so the K most probable tokens are the K
largest teacher logits ``z_iv = W_T[v] . h_i``.  Readings where the pages are
silent: the record lists them by logit, largest first; equal logits are
ordered by the lower token id first (which also decides which of several equal
logits at the K-th place is kept).

The plain definition, written out: for each row, all V logits (fp64 GEMM),
ordered by the key (-z, id), the first K kept.  Rows are processed in blocks
only to bound host memory.
"""
from __future__ import annotations

import numpy as np


def teacher_topk(H: np.ndarray, W: np.ndarray, k: int, block: int = 256):
    """(ids [n,k] int64, logits [n,k] float64) of the k largest ``H W^T`` per
    row, largest first, ties broken by the lower id.  H [n,d], W [v,d] fp64."""
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    n, v = H.shape[0], W.shape[0]
    if not 1 <= k <= v:
        raise ValueError("need 1 <= k <= v")
    ids = np.empty((n, k), dtype=np.int64)
    vals = np.empty((n, k), dtype=np.float64)
    cols = np.arange(v)
    for r0 in range(0, n, block):
        Z = H[r0:r0 + block] @ W.T
        for j, z in enumerate(Z):
            order = np.lexsort((cols, -z))[:k]  # primary key -z, then id
            ids[r0 + j] = order
            vals[r0 + j] = z[order]
    return ids, vals
