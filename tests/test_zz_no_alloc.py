"""GPU test of kd_chunked_fwd_noalloc, the forward that allocates nothing.

It runs the forward with the library's file-scope device scratch instead of
a caller workspace.  Its outputs must equal kd_chunked_fwd's bit for bit
(same kernels, same per-row arithmetic; the running loss adds chunk-sized
slices in order whatever the pass size).  Two calls in a row share the one
scratch array of the GPU, the second on a smaller input; the first problem is
sized so the scratch holds two chunks per pass while kd_chunked_fwd's
workspace holds eight, so the two entry points walk different passes.
"""
import pytest
import torch

from chunked_kl_loss_row_amd import binding as B
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, upload

pytestmark = pytest.mark.gpu


def _noalloc(d, chunk):
    prob = L.make_problem(d["H"], d["W"], d["t_ids"], d["t_logits"], chunk)
    n, k = prob.n, prob.k
    out = {"loss": torch.full((1,), float("nan"), device="cuda"),
           "lse": torch.full((n,), float("nan"), device="cuda"),
           "row_loss": torch.full((n,), float("nan"), device="cuda"),
           "zg": torch.full((n, k), float("nan"), device="cuda")}
    B.kd_chunked_fwd_noalloc(prob, d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], out["loss"], out["lse"],
                             out["row_loss"], out["zg"])
    return out


def _check_equal(d, chunk, tag):
    ref = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=chunk, row_loss=True, zg=True)
    got = _noalloc(d, chunk)
    torch.cuda.synchronize()
    log(f"[{tag}] loss workspace={float(ref['loss'].item()):.9g} noalloc={float(got['loss'].item()):.9g}")
    for key in ("loss", "lse", "row_loss", "zg"):
        assert torch.equal(got[key], ref[key]), key


def test_noalloc_forward_two_calls():
    # first call: 20000 rows, chunk 4096 -- about 25 MB of scratch per chunk, so two chunks per pass
    # (three passes), against one pass of eight chunks with the workspace
    wl1 = inputs.custom(20000, 2048, 32768, 100, 4096, x_dtype="bf16", w_std=0.02, mask="tail:300", tag=951)
    prob1 = B.problem(wl1.n, wl1.d, wl1.v, wl1.k, wl1.chunk, B.KD_BF16)
    log(f"case noalloc 1: {wl1.name} chunk={wl1.chunk}")
    d1 = upload(inputs.make_inputs(wl1, seed=0))
    assert B.kd_chunked_workspace_size(prob1) > 8 * 25 * 10 ** 6  # the workspace path takes larger passes
    _check_equal(d1, wl1.chunk, "noalloc 1")
    del d1
    # second call, smaller input (fp32, random mask): the scratch still holds the first call's data
    wl2 = inputs.custom(700, 192, 3000, 37, 300, x_dtype="f32", mask="random:50", tag=952)
    log(f"case noalloc 2: {wl2.name} chunk={wl2.chunk}")
    d2 = upload(inputs.make_inputs(wl2, seed=1))
    _check_equal(d2, wl2.chunk, "noalloc 2")
    # n = 0 writes a zero loss
    wl3 = inputs.custom(0, 64, 500, 8, 32, x_dtype="bf16")
    d3 = upload(inputs.make_inputs(wl3, seed=0))
    got = _noalloc(d3, 32)
    torch.cuda.synchronize()
    assert float(got["loss"].item()) == 0.0


def test_noalloc_forward_refuses_oversized_chunk():
    wl = inputs.custom(64, 64, 500, 8, 32, x_dtype="bf16")
    d = upload(inputs.make_inputs(wl, seed=0))
    prob = B.problem(64, 8192, 200000, 100, 4096, B.KD_BF16)  # one chunk needs ~86 MB of scratch
    loss = torch.full((1,), 7.0, device="cuda")
    st = B.kd_chunked_fwd_noalloc(prob, d["H"], d["W"], d["t_ids"], d["t_logits"], None, loss,
                                  torch.empty(64, device="cuda"), check=False)
    torch.cuda.synchronize()
    assert st == B.KD_ERR_WORKSPACE
    assert float(loss.item()) == 7.0  # nothing was enqueued
