"""GPU tests of the single-call path kd_chunked_fwd_bwd.

It keeps each chunk's fp32 logits from the forward projection and forms dZ
from them instead of recomputing the projection.  The kept logits are the
same fp32 values the recomputation produces, and dZ is formed with the same
formula, so loss, lse, dH and dW must equal those of kd_chunked_fwd followed
by kd_chunked_bwd bit for bit; one case is also checked against the fp64
oracle at the tolerances of the parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import binding as B
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, rel, rel_fro, upload

pytestmark = pytest.mark.gpu

CASES = [
    # n, d, v, k, chunk, x_dtype, mask, g
    (256, 128, 4096, 16, 64, "f32", "random:13", None),
    (700, 192, 3000, 37, 300, "bf16", "random:50", 0.37),
    (600, 520, 2000, 64, 256, "bf16", "tail:40", None),
    (257, 200, 777, 256, 100, "bf16", "none", -2.5),
    (1024, 384, 5000, 100, 512, "f32", "random:100", 1.0),
]


def _two_call(d, chunk, g, dW0):
    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=chunk)
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], f["lse"], g, dW=dW0.clone(),
                        chunk=chunk, workspace=f["workspace"])
    return f["loss"], f["lse"], dH, dW


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "x".join(map(str, s[:5])) + "-" + s[5])
def test_single_call_matches_two_calls_bitwise(spec):
    n, dd, v, k, chunk, xd, mask, g = spec
    wl = inputs.custom(n, dd, v, k, chunk, x_dtype=xd, mask=mask, tag=400 + n)
    log(f"case {wl.name} chunk={chunk} {xd} mask={mask} g={g}")
    inp = inputs.make_inputs(wl, seed=3)
    d = upload(inp)
    gl = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda")
    dW0 = torch.randn(v, dd, device="cuda")  # prior contents: both paths accumulate into it
    loss2, lse2, dH2, dW2 = _two_call(d, chunk, gl, dW0)
    f = L.forward_backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], gl, dW=dW0.clone(), chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(f["loss"], loss2)
    assert torch.equal(f["lse"], lse2)
    assert torch.equal(f["dH"], dH2)
    assert torch.equal(f["dW"], dW2)
    if mask != "none":
        masked = torch.from_numpy(np.nonzero(inp["mask"] == 0)[0]).cuda()
        assert bool((f["dH"][masked] == 0).all())


def test_single_call_against_oracle():
    wl = inputs.custom(700, 192, 3000, 37, 300, x_dtype="bf16", mask="random:50", tag=411)
    inp = inputs.make_inputs(wl, seed=4)
    d = upload(inp)
    gl = torch.tensor([0.37], dtype=torch.float32, device="cuda")
    f = L.forward_backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], gl, chunk=wl.chunk)
    torch.cuda.synchronize()
    ref = oracle.run(inp, g=0.37)
    loss = float(f["loss"].item())
    log(f"single call: loss gpu={loss:.9g} oracle={ref['loss']:.9g}")
    assert rel(loss, ref["loss"]) <= 1e-3
    np.testing.assert_allclose(f["lse"].cpu().numpy(), ref["lse"], rtol=1e-5, atol=0)
    assert rel_fro(f["dH"].cpu().numpy(), ref["dH"]) <= 1e-2
    assert rel_fro(f["dW"].cpu().numpy(), ref["dW"]) <= 1e-2


def test_single_call_workspace_and_empty():
    prob = B.problem(1000, 256, 5000, 100, 512, B.KD_BF16)
    base, fused = B.kd_chunked_workspace_size(prob), B.kd_chunked_fwd_bwd_workspace_size(prob)
    ldz = 384 * ((5000 + 383) // 384)
    assert fused >= base + 512 * ldz * 4
    # workspace never depends on n
    assert B.kd_chunked_fwd_bwd_workspace_size(B.problem(10 ** 7, 256, 5000, 100, 512, B.KD_BF16)) == fused
    # n = 0: loss 0, nothing else touched
    wl = inputs.custom(0, 64, 500, 8, 32, x_dtype="bf16")
    inp = inputs.make_inputs(wl, seed=0)
    d = upload(inp)
    f = L.forward_backward(d["H"], d["W"], d["t_ids"], d["t_logits"], None, chunk=32)
    torch.cuda.synchronize()
    assert float(f["loss"].item()) == 0.0
    # a workspace one byte short is refused before anything is enqueued
    wl = inputs.custom(64, 64, 500, 8, 32, x_dtype="bf16")
    d = upload(inputs.make_inputs(wl, seed=0))
    p2 = L.make_problem(d["H"], d["W"], d["t_ids"], d["t_logits"], 32)
    need = B.kd_chunked_fwd_bwd_workspace_size(p2)
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    st = B.kd_chunked_fwd_bwd(p2, d["H"], d["W"], d["t_ids"], d["t_logits"], None, None,
                              torch.empty(1, device="cuda"), torch.empty(64, device="cuda"),
                              torch.empty(64, 64, device="cuda"), torch.zeros(500, 64, device="cuda"), ws,
                              check=False)
    assert st == B.KD_ERR_WORKSPACE
