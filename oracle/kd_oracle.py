"""fp64 CPU oracle of the top-K KL distillation loss (test infrastructure).

TEST INFRASTRUCTURE ONLY.  This module may be imported, called or executed by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` -- nothing else.  The HIP library and its Python binding never
import it, and it imports nothing from them.

What it computes
----------------
The pages compare three ways of computing one and the same distillation loss
(dense, forward-chunked, fused chunked) and state that they are mathematically
equivalent (aihot.vn page "Tối ưu hóa chi phí chưng cất tri thức…", section
"Hai thay đổi hệ thống"; aifeed.pl page "Destylacja wiedzy AI taniej o 50%…",
section "Dwie kluczowe zmiany systemowe").  The oracle is therefore the plain
dense definition -- the "textbook" variant that builds the full
vocabulary-by-position grid -- written out in fp64 with numpy:

* teacher: the cached record per position is K token ids and K teacher logits
  (the 100 most probable tokens, agentlenshq.com page
  "LLMのための効率的な知識蒸留…", section
  "1. Top-K Logit Cachingによるオフライン蒸留").  Reading: the teacher
  distribution is the softmax of those K logits, renormalised over the K
  entries, no bucket for the remaining mass.
* student: logits ``z_i = W h_i`` over the full vocabulary (the loss owns the
  output projection: agentlenshq.com page, section "2. Fused Chunked KL Loss"),
  log-probabilities ``log q_iv = z_iv - lse_i`` normalised over all V.
* loss: reading: forward KL(teacher || student) restricted to the K cached ids,
  summed over unmasked positions:
  ``L = sum_i m_i sum_k p_ik (log p_ik - z_{i,t_ik} + lse_i)``.
  Reading for records that break the cache's contract (ids outside [0, V)):
  such an id matches no vocabulary entry -- its gathered logit ``z_{i,t_ik}``
  is taken as 0 and it adds no term to dZ, while its ``p_ik`` still counts in
  ``sum_k p_ik`` and ``sum_k p_ik log p_ik``.
* gradient: the pages mention, without printing it, a closed-form gradient
  behind the fused chunked loss (aihot.vn page, section "Mô hình học sinh thu
  được").  From the definition above,
  ``dL/dz_iv = g m_i (s_i q_iv - sum_k p_ik [t_ik = v])`` with
  ``s_i = sum_k p_ik``; then ``dH = dZ W`` and ``dW = dZ^T H``.
* temperature, a loss variant: the aihot.vn page (section "Mô hình học sinh
  thu được") reports ablations over the choice of loss without defining any;
  reading: the usual temperature-scaled distillation loss.
  Teacher ``p = softmax(a / tau)`` over the K entries, student
  ``q = softmax(z / tau)`` over V, ``L = tau^2 sum_i m_i KL(p_i || q_i)`` at
  the K ids; ``lse_i = log sum_v exp(z_iv / tau)``; the gathered logits stay
  ``z``; ``dL/dz_iv = g tau m_i (s_i q_iv - sum_k p_ik [t_ik = v])``.
  ``tau = 1`` is the loss above.

Rows are processed in blocks only to bound host memory; rows are independent,
so the blocking does not change any value beyond fp64 rounding order of the
library GEMM (which does not depend on the block for a given row).

Inputs arrive as the stored values (bf16 bit patterns as uint16, or float32);
they are widened exactly to fp64 here.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# exact widening of stored inputs
# ----------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input -> float64, exactly (bf16 bits are the top half of an fp32)."""
    if dtype == "bf16":
        x = np.asarray(x)
        if x.dtype != np.uint16:
            raise TypeError("bf16 inputs are passed as uint16 bit patterns")
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# teacher side
# ----------------------------------------------------------------------------
def teacher_distribution(t_logits: np.ndarray, tau: float = 1.0):
    """Renormalised top-K teacher distribution of each row.

    ``p_ik = exp(a_ik - max_j a_ij) / sum_j exp(a_ij - max_j a_ij)`` with the
    logits divided by ``tau`` first; returns ``p [n,K]``,
    ``negent [n] = sum_k p_ik log p_ik`` (``0 log 0 = 0``) and
    ``s [n] = sum_k p_ik``.  Cached top-K record: agentlenshq.com page,
    section "1. Top-K Logit Cachingによるオフライン蒸留"."""
    a = np.asarray(t_logits, dtype=np.float64) / tau
    amax = a.max(axis=1, keepdims=True)
    e = np.exp(a - amax)
    p = e / e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0.0, p * np.log(p), 0.0)
    return p, plogp.sum(axis=1), p.sum(axis=1)


# ----------------------------------------------------------------------------
# student side
# ----------------------------------------------------------------------------
def student_logits(h_rows: np.ndarray, w: np.ndarray) -> np.ndarray:
    """``Z = H_rows W^T`` in fp64 (the output projection the loss owns)."""
    return h_rows @ w.T


def row_logsumexp(z: np.ndarray) -> np.ndarray:
    """``lse_i = log sum_v exp z_iv`` over the full vocabulary (max-shifted)."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


# ----------------------------------------------------------------------------
# forward: loss, lse, gathered logits, per-row loss
# ----------------------------------------------------------------------------
def _mask_rows(mask: Optional[np.ndarray], rows: np.ndarray) -> np.ndarray:
    if mask is None:
        return np.ones(rows.size, dtype=np.float64)
    return (np.asarray(mask)[rows] != 0).astype(np.float64)


def kd_forward(H: np.ndarray, W: np.ndarray, t_ids: np.ndarray, t_logits: np.ndarray,
               mask: Optional[np.ndarray] = None, rows: Optional[Sequence[int]] = None,
               block: int = 256, tau: float = 1.0) -> dict:
    """Dense forward on fp64 inputs (already widened).

    ``rows`` restricts the evaluation to a subset of positions (rows are
    independent); ``loss`` is then the sum over that subset.  Masked rows
    contribute 0 and their teacher record is not read.
    Returns ``loss`` (python float, summed with ``math.fsum``), ``lse`` (of
    ``z / tau``), ``zg [r,K]`` (the logits ``z`` at the ids), ``row_loss``."""
    n = H.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    K = t_ids.shape[1]
    m = _mask_rows(mask, rows)
    lse = np.empty(rows.size)
    zg = np.zeros((rows.size, K))
    row_loss = np.zeros(rows.size)
    for b0 in range(0, rows.size, block):
        sel = rows[b0:b0 + block]
        z = student_logits(H[sel], W)
        lse_b = row_logsumexp(z / tau)
        lse[b0:b0 + sel.size] = lse_b
        live = m[b0:b0 + sel.size] != 0
        if not live.any():
            continue
        li = np.nonzero(live)[0]
        ids = np.asarray(t_ids[sel[li]], dtype=np.int64)
        # an id outside [0, V) matches no vocabulary entry: its gathered logit is 0
        inside = (ids >= 0) & (ids < z.shape[1])
        zg_b = np.where(inside, np.take_along_axis(z[li], np.where(inside, ids, 0), axis=1), 0.0)
        p, negent, s = teacher_distribution(t_logits[sel[li]], tau)
        zg[b0 + li] = zg_b
        # tau^2 sum_k p (log p - (z_t / tau - lse)) = tau^2 (negent - sum_k p z_t / tau + s * lse)
        row_loss[b0 + li] = tau * tau * (negent - (p * zg_b).sum(axis=1) / tau + s * lse_b[li])
    return {"loss": math.fsum(row_loss.tolist()), "lse": lse, "zg": zg,
            "row_loss": row_loss, "rows": rows}


# ----------------------------------------------------------------------------
# backward: closed-form dZ, dH, dW
# ----------------------------------------------------------------------------
def kd_backward(H: np.ndarray, W: np.ndarray, t_ids: np.ndarray, t_logits: np.ndarray,
                mask: Optional[np.ndarray] = None, g: float = 1.0,
                rows: Optional[Sequence[int]] = None, want_dw: bool = True,
                want_dz: bool = False, block: int = 256, tau: float = 1.0) -> dict:
    """Gradient of ``g * L`` for the positions in ``rows`` (default: all).

    ``dZ_iv = g tau m_i (s_i exp(z_iv / tau - lse_i) - sum_k p_ik [t_ik = v])``;
    ``dH_i = dZ_i W`` (one row per requested position) and
    ``dW = sum_{i in rows} dZ_i^T h_i`` (the contribution of those rows; equal
    to the full dW when the mask is zero outside them).  The p-scatter uses
    ``np.add.at`` so repeated ids in a row add term by term."""
    n, D = H.shape
    V = W.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    m = _mask_rows(mask, rows)
    dH = np.zeros((rows.size, D))
    dW = np.zeros((V, D)) if want_dw else None
    dZ_all = np.zeros((rows.size, V)) if want_dz else None
    for b0 in range(0, rows.size, block):
        sel = rows[b0:b0 + block]
        mb = m[b0:b0 + sel.size]
        live = np.nonzero(mb != 0)[0]
        if live.size == 0:
            continue
        hs = H[sel[live]]
        z = student_logits(hs, W) / tau
        lse_b = row_logsumexp(z)
        p, _, s = teacher_distribution(t_logits[sel[live]], tau)
        dz = s[:, None] * np.exp(z - lse_b[:, None])
        ids_b = np.asarray(t_ids[sel[live]], dtype=np.int64).ravel()
        inside = (ids_b >= 0) & (ids_b < V)  # an id outside [0, V) matches no column
        r_idx = np.repeat(np.arange(live.size), p.shape[1])
        np.add.at(dz, (r_idx[inside], ids_b[inside]), -p.ravel()[inside])
        dz *= g * tau
        dH[b0 + live] = dz @ W
        if want_dw:
            dW += dz.T @ hs
        if want_dz:
            dZ_all[b0 + live] = dz
    out = {"dH": dH, "rows": rows}
    if want_dw:
        out["dW"] = dW
    if want_dz:
        out["dZ"] = dZ_all
    return out


def dw_vocab_rows(H_stored, W_stored, x_dtype: str, t_ids: np.ndarray, t_logits: np.ndarray,
                  mask: Optional[np.ndarray], lse: np.ndarray, vocab: Sequence[int], g: float = 1.0,
                  tau: float = 1.0, block: int = 4096) -> np.ndarray:
    """Rows ``vocab`` (distinct ids) of ``dW`` summed over ALL positions, given
    each row's ``lse`` (of ``z / tau`` over the full vocabulary).

    The closed form of ``kd_backward`` restricted to the requested vocabulary
    columns of dZ: ``dW_u = sum_i dZ_iu h_i`` with
    ``dZ_iu = g tau m_i (s_i exp(z_iu / tau - lse_i) - sum_k p_ik [t_ik = u])``.
    Because ``lse`` is given, only the requested columns of z are formed, so a
    full-size problem fits in host memory.  ``H_stored`` / ``W_stored`` are the
    stored inputs (``x_dtype`` as for ``widen``); H is widened block by block."""
    vocab = np.asarray(vocab, dtype=np.int64)
    if np.unique(vocab).size != vocab.size:
        raise ValueError("vocab ids must be distinct")
    n = H_stored.shape[0]
    V = W_stored.shape[0]
    Wv = widen(W_stored[vocab], x_dtype)                # [U, D]
    col = np.full(V, -1, dtype=np.int64)
    col[vocab] = np.arange(vocab.size)
    lse = np.asarray(lse, dtype=np.float64)
    out = np.zeros((vocab.size, Wv.shape[1]))
    live_all = np.nonzero(_mask_rows(mask, np.arange(n)) != 0)[0]
    for b0 in range(0, live_all.size, block):
        live = live_all[b0:b0 + block]
        hs = widen(H_stored[live], x_dtype)
        z = student_logits(hs, Wv) / tau                # [r, U]
        p, _, s = teacher_distribution(t_logits[live], tau)
        dz = s[:, None] * np.exp(z - lse[live][:, None])
        ids = np.asarray(t_ids[live], dtype=np.int64)
        inside = (ids >= 0) & (ids < V)
        j = np.where(inside, col[np.clip(ids, 0, V - 1)], -1)
        r, kk = np.nonzero(j >= 0)
        np.add.at(dz, (r, j[r, kk]), -p[r, kk])
        out += (g * tau) * (dz.T @ hs)
    return out


# ----------------------------------------------------------------------------
# convenience: widen a stored input dict and run both passes
# ----------------------------------------------------------------------------
def widen_inputs(inp: dict) -> dict:
    """Widen the stored arrays of an input dict (``H``, ``W``, ``t_logits``)."""
    wl = inp["wl"]
    return {
        "H": widen(inp["H"], wl.x_dtype),
        "W": widen(inp["W"], wl.x_dtype),
        "t_ids": np.asarray(inp["t_ids"]),
        "t_logits": widen(inp["t_logits"], wl.t_dtype),
        "mask": inp["mask"],
    }


def run(inp: dict, g: float = 1.0, rows=None, want_dw: bool = True, block: int = 256,
        tau: float = 1.0) -> dict:
    """Forward and backward of one stored input dict, all in fp64."""
    x = widen_inputs(inp)
    f = kd_forward(x["H"], x["W"], x["t_ids"], x["t_logits"], x["mask"], rows=rows, block=block, tau=tau)
    b = kd_backward(x["H"], x["W"], x["t_ids"], x["t_logits"], x["mask"], g=g, rows=rows,
                    want_dw=want_dw, block=block, tau=tau)
    f.update(b)
    return f
