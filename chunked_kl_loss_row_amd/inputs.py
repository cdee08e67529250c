"""Seeded synthetic inputs for the fused chunked top-K KL loss.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the loss's arithmetic.  Both the HIP path (through the binding) and the
fp64 oracle are fed from it, and nothing else is shared between them.

The pages measure on model training runs whose weights and corpora are not
available; these draws stand in for them with the workload shapes below:

* hidden states ``H ~ N(0, 1)``, output projection ``W ~ N(0, sigma_w^2)``;
* a cached teacher record per position: ``K`` distinct token ids and ``K``
  teacher logits ``~ N(0, sigma_t^2)`` sorted in descending order (the pages
  cache the 100 most probable tokens per position: agentlenshq.com page
  "LLMのための効率的な知識蒸留…", section "1. Top-K Logit Cachingによるオフライン蒸留");
* an optional per-position mask (padding).

Storage: ``bf16`` arrays are returned as ``uint16`` bit patterns (round to
nearest even from float32), ``f32`` arrays as ``float32``.  Random streams come
from ``numpy.random.Generator(PCG64(SeedSequence([tag, seed, stream])))``, one
stream per tensor, so every tensor can be regenerated independently.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# stream ids (one PCG64 stream per tensor)
_S_H, _S_W, _S_IDS, _S_LOGITS, _S_MASK, _S_HOT = range(6)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""

    name: str
    n: int                 # positions (batch * seq, flattened)
    d: int                 # hidden size
    v: int                 # vocabulary size
    k: int                 # teacher top-K
    chunk: int             # rows per chunk
    x_dtype: str           # "f32" | "bf16": dtype of H and W
    t_dtype: str           # "f32" | "bf16": dtype of teacher logits
    w_std: float           # std of W entries (None -> 1/sqrt(d))
    logit_std: float       # std of teacher logits
    mask: str = "none"     # "none" | "random:<count>" | "tail:<count>"
    ids: str = "uniform"   # "uniform" | "hot:<batch>:<hot>:<from_hot>"
    tag: int = 0           # seed-sequence tag (workload index)


# Workloads: index 0 is the tiny fp32 case, 1..4 the gpt-oss / Llama shapes.
WORKLOADS = [
    Workload("tiny-f32", n=256, d=128, v=4096, k=16, chunk=64, x_dtype="f32",
             t_dtype="f32", w_std=1.0 / np.sqrt(128.0), logit_std=2.0,
             mask="random:13", tag=1),
    Workload("llama3.2-3b-8k", n=8192, d=3072, v=128256, k=100, chunk=1024,
             x_dtype="bf16", t_dtype="bf16", w_std=0.02, logit_std=3.0, tag=2),
    Workload("gpt-oss-20b-32k", n=32768, d=2880, v=201088, k=100, chunk=2048,
             x_dtype="bf16", t_dtype="bf16", w_std=0.02, logit_std=3.0,
             mask="tail:983", tag=3),
    Workload("gpt-oss-120b-b4x32k", n=131072, d=2880, v=201088, k=100,
             chunk=2048, x_dtype="bf16", t_dtype="bf16", w_std=0.02,
             logit_std=3.0, ids="hot:4:4096:70", tag=4),
    Workload("long-256k", n=262144, d=4096, v=128256, k=100, chunk=4096,
             x_dtype="bf16", t_dtype="bf16", w_std=0.02, logit_std=3.0, tag=5),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def custom(n, d, v, k, chunk, x_dtype="bf16", t_dtype=None, w_std=None,
           logit_std=3.0, mask="none", ids="uniform", tag=100) -> Workload:
    """A small workload for tests (several tiles, ragged tails)."""
    return Workload(f"custom-{n}x{d}x{v}x{k}", n=n, d=d, v=v, k=k, chunk=chunk,
                    x_dtype=x_dtype, t_dtype=t_dtype or x_dtype,
                    w_std=(1.0 / np.sqrt(d)) if w_std is None else w_std,
                    logit_std=logit_std, mask=mask, ids=ids, tag=tag)


def _rng(tag: int, seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([tag, seed, stream])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + (0x7FFF + ((u >> 16) & 1))) >> 16
    out = rounded.astype(np.uint16)
    out[is_nan] = ((u[is_nan] >> 16) | 0x0040).astype(np.uint16)  # keep NaN quiet
    return out


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(dtype)


def _normal_rows(rng, n, d, std, dtype, block=8192):
    """N(0, std^2) matrix [n, d] drawn in row blocks, stored in ``dtype``."""
    out = np.empty((n, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        x = rng.standard_normal((r1 - r0, d), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[r0:r1] = _store(x, dtype)
    return out


def _distinct_rows(rng, n, k, lo, hi):
    """[n, k] int64 ids, each row ``k`` distinct values uniform in [lo, hi).

    Draw with replacement, then redraw every row that holds a repeat (rows
    without repeats keep their draw order, so the ids are not sorted)."""
    if hi - lo < k:
        raise ValueError("not enough ids for k distinct draws")
    if k * k > 2 * (hi - lo):
        # many repeats expected: take the first k entries of a random
        # permutation of the range per row instead
        keys = rng.random((n, hi - lo))
        return np.argsort(keys, axis=1)[:, :k].astype(np.int64) + lo
    ids = rng.integers(lo, hi, size=(n, k), dtype=np.int64)
    todo = np.arange(n)
    while True:
        s = np.sort(ids[todo], axis=1)
        bad = todo[(s[:, 1:] == s[:, :-1]).any(axis=1)] if k > 1 else todo[:0]
        if bad.size == 0:
            return ids
        ids[bad] = rng.integers(lo, hi, size=(bad.size, k), dtype=np.int64)
        todo = bad


def _teacher_ids(wl: Workload, seed: int, n: int) -> np.ndarray:
    rng = _rng(wl.tag, seed, _S_IDS)
    if wl.ids == "uniform":
        out = np.empty((n, wl.k), dtype=np.int32)
        block = 16384
        for r0 in range(0, n, block):
            r1 = min(n, r0 + block)
            out[r0:r1] = _distinct_rows(rng, r1 - r0, wl.k, 0, wl.v)
        return out
    if wl.ids.startswith("hot:"):
        # per sequence: a hot set of `hot` distinct ids; each row takes exactly
        # `from_hot` distinct ids from it and the rest distinct from outside it,
        # shuffled within the row (skewed id reuse across positions).
        _, nb, hot, from_hot = wl.ids.split(":")
        nb, hot, from_hot = int(nb), int(hot), int(from_hot)
        rest = wl.k - from_hot
        rhot = _rng(wl.tag, seed, _S_HOT)
        out = np.empty((n, wl.k), dtype=np.int32)
        seq = -(-n // nb)
        for b in range(nb):
            r0, r1 = b * seq, min(n, (b + 1) * seq)
            if r0 >= r1:
                break
            hot_ids = rhot.permutation(wl.v)[:hot]
            cold = np.setdiff1d(np.arange(wl.v), hot_ids)  # sorted complement
            for q0 in range(r0, r1, 16384):
                q1 = min(r1, q0 + 16384)
                h = hot_ids[_distinct_rows(rng, q1 - q0, from_hot, 0, hot)]
                c = cold[_distinct_rows(rng, q1 - q0, rest, 0, cold.size)]
                both = np.concatenate([h, c], axis=1)
                out[q0:q1] = rng.permuted(both, axis=1)
        return out
    raise ValueError(wl.ids)


def _teacher_logits(wl: Workload, seed: int, n: int) -> np.ndarray:
    rng = _rng(wl.tag, seed, _S_LOGITS)
    out = np.empty((n, wl.k), dtype=np.uint16 if wl.t_dtype == "bf16" else np.float32)
    for r0 in range(0, n, 65536):
        r1 = min(n, r0 + 65536)
        x = rng.standard_normal((r1 - r0, wl.k), dtype=np.float32) * np.float32(wl.logit_std)
        x = -np.sort(-x, axis=1)  # descending
        out[r0:r1] = _store(x, wl.t_dtype)
    return out


def _mask(wl: Workload, seed: int, n: int) -> Optional[np.ndarray]:
    if wl.mask == "none":
        return None
    kind, cnt = wl.mask.split(":")
    cnt = int(cnt)
    m = np.ones(n, dtype=np.uint8)
    if kind == "random":
        rng = _rng(wl.tag, seed, _S_MASK)
        m[rng.choice(n, size=min(cnt, n), replace=False)] = 0
    elif kind == "tail":
        if cnt > 0:
            m[max(0, n - cnt):] = 0
    else:
        raise ValueError(wl.mask)
    return m


def make_inputs(wl: Workload, seed: int = 0, n: Optional[int] = None,
                only: Optional[tuple] = None) -> dict:
    """All inputs of one workload as host numpy arrays.

    Returns a dict with ``H [n,d]``, ``W [v,d]`` (uint16 bf16 bits or float32),
    ``t_ids [n,k] int32``, ``t_logits [n,k]`` (bits or float32), ``mask``
    (``[n] uint8`` or ``None``) and the workload itself under ``wl``.
    ``n`` overrides the number of positions (same recipe, fewer rows);
    ``only`` names a subset of the tensors to draw (each has its own stream,
    so the others are unaffected)."""
    n = wl.n if n is None else int(n)
    want = set(only) if only is not None else {"H", "W", "t_ids", "t_logits", "mask"}
    out = {"wl": wl, "n": n}
    if "H" in want:
        out["H"] = _normal_rows(_rng(wl.tag, seed, _S_H), n, wl.d, 1.0, wl.x_dtype)
    if "W" in want:
        out["W"] = _normal_rows(_rng(wl.tag, seed, _S_W), wl.v, wl.d, wl.w_std, wl.x_dtype)
    if "t_ids" in want:
        out["t_ids"] = _teacher_ids(wl, seed, n)
    if "t_logits" in want:
        out["t_logits"] = _teacher_logits(wl, seed, n)
    if "mask" in want:
        out["mask"] = _mask(wl, seed, n)
    return out


def sample_rows(n: int, count: int, seed: int = 0, tag: int = 999) -> np.ndarray:
    """Seeded sorted subset of ``count`` distinct row indices in [0, n)."""
    rng = _rng(tag, seed, 0)
    count = min(count, n)
    return np.sort(rng.choice(n, size=count, replace=False)).astype(np.int64)
