"""torch-facing wrapper of the fused chunked top-K KL loss.

PyTorch supplies device memory, the current stream and autograd plumbing;
every arithmetic step runs in libkdchunk.so through ``binding``.

    loss = kd_chunked_kl(hidden, weight, t_ids, t_logits, mask=None, chunk=2048)
    loss.backward()      # hidden.grad (fp32), weight.grad (fp32 accumulator)

The loss is the sum over unmasked positions of KL(teacher top-K, renormalised
|| student softmax over the full vocabulary) at the K cached ids; the
projection ``hidden @ weight.T`` is fused into it and computed one chunk of
positions at a time, recomputed in the backward pass (agentlenshq.com page
"LLMのための効率的な知識蒸留…", section "2. Fused Chunked KL Loss").
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B


def _xdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return B.KD_BF16
    if t.dtype == torch.float32:
        return B.KD_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def make_problem(hidden, weight, t_ids, t_logits, chunk: int, temperature: float = 1.0,
                 dw_chunks: int = 1) -> B.KDProblem:
    n, d = hidden.shape
    v, d2 = weight.shape
    if d2 != d:
        raise ValueError("hidden and weight disagree on the hidden size")
    if t_ids.shape != t_logits.shape or t_ids.shape[0] != n:
        raise ValueError("teacher ids / logits must be [n, k]")
    if hidden.dtype != weight.dtype:
        raise TypeError("hidden and weight must share a dtype")
    if t_ids.dtype != torch.int32:
        raise TypeError("teacher ids must be int32")
    return B.problem(n, d, v, t_ids.shape[1], chunk, _xdtype(hidden), _xdtype(t_logits), temperature, dw_chunks)


def _check_mask(mask, n):
    if mask is not None and (mask.dtype not in (torch.uint8, torch.bool) or mask.shape != (n,)):
        raise TypeError("mask must be a uint8 (or bool) tensor of shape [n]")


def _check(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def workspace_for(prob: B.KDProblem, device) -> torch.Tensor:
    return torch.empty(B.kd_chunked_workspace_size(prob), dtype=torch.uint8, device=device)


def forward(hidden, weight, t_ids, t_logits, mask=None, chunk: int = 2048, workspace=None,
            row_loss: bool = False, zg: bool = False, temperature: float = 1.0, dw_chunks: int = 1) -> dict:
    """Run kd_chunked_fwd; returns {"loss", "lse", "row_loss"?, "zg"?, "workspace"}.  ``dw_chunks``
    only sizes the workspace (it must match the backward's when the workspace is shared)."""
    _check(hidden, weight, t_ids, t_logits, mask)
    prob = make_problem(hidden, weight, t_ids, t_logits, chunk, temperature, dw_chunks)
    _check_mask(mask, prob.n)
    dev = hidden.device
    ws = workspace if workspace is not None else workspace_for(prob, dev)
    out = {"loss": torch.empty(1, dtype=torch.float32, device=dev),
           "lse": torch.empty(prob.n, dtype=torch.float32, device=dev),
           "row_loss": torch.empty(prob.n, dtype=torch.float32, device=dev) if row_loss else None,
           "zg": torch.empty(prob.n, prob.k, dtype=torch.float32, device=dev) if zg else None,
           "workspace": ws}
    B.kd_chunked_fwd(prob, hidden, weight, t_ids, t_logits, mask, out["loss"], out["lse"],
                     out["row_loss"], out["zg"], ws)
    return out


def backward(hidden, weight, t_ids, t_logits, mask, lse, grad_loss=None, dW=None, chunk: int = 2048,
             workspace=None, dH=None, temperature: float = 1.0, dw_chunks: int = 1):
    """Run kd_chunked_bwd; returns (dH, dW).  ``dW`` (fp32) is accumulated
    into when given, else a zero buffer is made.  ``temperature`` must be the
    forward's.  ``dw_chunks`` chunks of dZ feed one dW GEMM (more workspace,
    fewer passes over dW)."""
    _check(hidden, weight, t_ids, t_logits, mask, lse, grad_loss)
    prob = make_problem(hidden, weight, t_ids, t_logits, chunk, temperature, dw_chunks)
    _check_mask(mask, prob.n)
    dev = hidden.device
    ws = workspace if workspace is not None else workspace_for(prob, dev)
    if dH is None:
        dH = torch.empty(prob.n, prob.d, dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.zeros(prob.v, prob.d, dtype=torch.float32, device=dev)
    if dW.dtype != torch.float32 or dH.dtype != torch.float32:
        raise TypeError("gradients are fp32")
    B.kd_chunked_bwd(prob, hidden, weight, t_ids, t_logits, mask, lse, grad_loss, dH, dW, ws)
    return dH, dW


def forward_backward(hidden, weight, t_ids, t_logits, mask=None, grad_loss=None, dW=None,
                     chunk: int = 2048, workspace=None, dH=None, temperature: float = 1.0,
                     dw_chunks: int = 1) -> dict:
    """kd_chunked_fwd_bwd: loss, lse, dH and dW (accumulated into ``dW`` when
    given) in one call, each chunk's logits kept instead of recomputed.
    Returns {"loss", "lse", "dH", "dW", "workspace"}."""
    _check(hidden, weight, t_ids, t_logits, mask, grad_loss)
    prob = make_problem(hidden, weight, t_ids, t_logits, chunk, temperature, dw_chunks)
    _check_mask(mask, prob.n)
    dev = hidden.device
    ws = workspace if workspace is not None else torch.empty(B.kd_chunked_fwd_bwd_workspace_size(prob),
                                                             dtype=torch.uint8, device=dev)
    out = {"loss": torch.empty(1, dtype=torch.float32, device=dev),
           "lse": torch.empty(prob.n, dtype=torch.float32, device=dev),
           "dH": dH if dH is not None else torch.empty(prob.n, prob.d, dtype=torch.float32, device=dev),
           "dW": dW if dW is not None else torch.zeros(prob.v, prob.d, dtype=torch.float32, device=dev),
           "workspace": ws}
    B.kd_chunked_fwd_bwd(prob, hidden, weight, t_ids, t_logits, mask, grad_loss, out["loss"], out["lse"],
                         out["dH"], out["dW"], ws)
    return out


def teacher_topk(hidden, weight, k: int = 100, chunk: int = 2048, workspace=None) -> dict:
    """kd_teacher_topk: the K largest logits of ``hidden @ weight.T`` per row
    (ids int32, fp32 logits, largest first, ties by the lower id).  Returns
    {"ids", "logits", "overflow_rows" (device int), "workspace"}."""
    _check(hidden, weight)
    n, d = hidden.shape
    v = weight.shape[0]
    if weight.shape[1] != d or hidden.dtype != weight.dtype:
        raise ValueError("hidden [n,d] and weight [v,d] of one dtype")
    prob = B.problem(n, d, v, k, chunk, _xdtype(hidden))
    dev = hidden.device
    ws = workspace if workspace is not None else torch.empty(B.kd_teacher_topk_workspace_size(prob),
                                                             dtype=torch.uint8, device=dev)
    out = {"ids": torch.empty(n, k, dtype=torch.int32, device=dev),
           "logits": torch.empty(n, k, dtype=torch.float32, device=dev),
           "overflow_rows": torch.zeros(1, dtype=torch.int32, device=dev), "workspace": ws}
    B.kd_teacher_topk(prob, hidden, weight, out["ids"], out["logits"], out["overflow_rows"], ws)
    return out


def validate_teacher(t_ids, v: int, mask=None) -> torch.Tensor:
    """kd_chunked_validate: checks the teacher record's ids (int32 [n, k])
    against the vocabulary size ``v`` on unmasked rows.  Returns an int64 [4]
    device tensor (no synchronisation): rows with an id outside [0, v), rows
    with a repeated id, and the first row of each kind (-1 if none)."""
    _check(t_ids, mask)
    if t_ids.dtype != torch.int32 or t_ids.dim() != 2:
        raise TypeError("teacher ids must be an int32 tensor [n, k]")
    n, k = t_ids.shape
    _check_mask(mask, n)
    out = torch.empty(4, dtype=torch.int64, device=t_ids.device)
    # d, chunk and the dtypes play no part in the check; any valid values do
    prob = B.problem(n, 8, v, k, 1, B.KD_F32)
    B.kd_chunked_validate(prob, t_ids, mask.view(torch.uint8) if mask is not None else None, out)
    return out


class KDChunkedKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, t_ids, t_logits, mask, chunk, temperature):
        out = forward(hidden, weight, t_ids, t_logits, mask, chunk, temperature=temperature)
        ctx.save_for_backward(hidden, weight, t_ids, t_logits, mask, out["lse"])
        ctx.chunk = chunk
        ctx.temperature = temperature
        ctx.workspace = out["workspace"]
        return out["loss"][0]

    @staticmethod
    def backward(ctx, g):
        hidden, weight, t_ids, t_logits, mask, lse = ctx.saved_tensors
        gl = g.reshape(1).to(torch.float32).contiguous()
        dH, dW = backward(hidden, weight, t_ids, t_logits, mask, lse, gl, chunk=ctx.chunk,
                          workspace=ctx.workspace, temperature=ctx.temperature)
        ctx.workspace = None
        gh = dH if hidden.dtype == torch.float32 else dH.to(hidden.dtype)
        gw = dW if weight.dtype == torch.float32 else dW.to(weight.dtype)
        return gh, gw, None, None, None, None, None


def kd_chunked_kl(hidden, weight, t_ids, t_logits, mask=None, chunk: int = 2048, temperature: float = 1.0):
    """0-d fp32 loss; differentiable w.r.t. ``hidden`` and ``weight``.
    ``temperature`` tau: tau^2 KL(softmax(a / tau) || softmax(z / tau)) at the
    K ids (1: the plain loss)."""
    return KDChunkedKL.apply(hidden, weight, t_ids, t_logits, mask, chunk, temperature)
