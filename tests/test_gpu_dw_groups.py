"""GPU tests of dW formed over groups of chunks (kd_problem.dw_chunks).

Grouping changes only which dZ rows one dW GEMM reads (the chunks of a group,
back to back), so:
  * loss, lse and dH equal the per-chunk path (dw_chunks = 1) bit for bit;
  * dW matches the oracle at the usual tolerances (fp32 1e-5, bf16 1e-2
    relative Frobenius) and the per-chunk dW to fp32 summation-order error;
  * the single-call path equals the two-call path bit for bit at the same
    grouping; prior dW contents are kept.
Shapes include ragged last groups and a chunk size that is not a multiple of
8 (a group's second chunk then starts at an unaligned column of H^T).
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, rel, rel_fro, upload

pytestmark = pytest.mark.gpu


def _run(d, chunk, groups, g=0.37, dW0=None):
    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=chunk, dw_chunks=groups)
    gl = torch.tensor([g], dtype=torch.float32, device="cuda")
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], f["lse"], gl,
                        dW=None if dW0 is None else dW0.clone(), chunk=chunk, workspace=f["workspace"],
                        dw_chunks=groups)
    torch.cuda.synchronize()
    return float(f["loss"].item()), f["lse"], dH, dW


CASES = [
    # n, d, v, k, chunk, x_dtype, mask, dw_chunks
    (1000, 136, 3000, 40, 128, "bf16", "random:60", 2),
    (1000, 136, 3000, 40, 128, "bf16", "random:60", 3),
    (450, 64, 1500, 16, 100, "f32", "tail:30", 2),
    (450, 64, 1500, 16, 100, "f32", "none", 8),
    (700, 192, 2000, 37, 256, "bf16", "none", 4),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "x".join(map(str, s[:5])) + f"-{s[5]}-g{s[7]}")
def test_grouped_dw(spec):
    n, dd, v, k, chunk, xd, mask, groups = spec
    wl = inputs.custom(n, dd, v, k, chunk, x_dtype=xd, mask=mask, tag=900 + n + groups)
    inp = inputs.make_inputs(wl, seed=8)
    d = upload(inp)
    log(f"case {wl.name} chunk={chunk} {xd} dw_chunks={groups}")
    loss1, lse1, dH1, dW1 = _run(d, chunk, 1)
    lossg, lseg, dHg, dWg = _run(d, chunk, groups)
    assert lossg == loss1 and torch.equal(lseg, lse1) and torch.equal(dHg, dH1)
    e_same = rel_fro(dWg.cpu().numpy(), dW1.cpu().numpy())
    ref = oracle.run(inp, g=0.37)
    tol = 1e-5 if xd == "f32" else 1e-2
    e_ref = rel_fro(dWg.cpu().numpy(), ref["dW"])
    log(f"[{wl.name} g={groups}] dW vs per-chunk {e_same:.3g}, vs oracle {e_ref:.3g}")
    assert e_same <= 1e-5 and e_ref <= tol
    assert rel(lossg, ref["loss"]) <= (1e-5 if xd == "f32" else 1e-3)


def test_grouped_dw_keeps_prior_contents():
    wl = inputs.custom(600, 128, 2000, 30, 128, x_dtype="bf16", tag=950)
    d = upload(inputs.make_inputs(wl, seed=9))
    prior = torch.randn(wl.v, wl.d, device="cuda")
    log("case grouped dW prior contents")
    _, _, _, base = _run(d, 128, 3)
    _, _, _, acc = _run(d, 128, 3, dW0=prior)
    torch.testing.assert_close(acc, prior + base, rtol=1e-5, atol=1e-5)


# chunk 100: the chunks of a group start inside dZ's 32-row blocks (the
# single-call path writes each chunk's dZ rows after the previous chunk's)
@pytest.mark.parametrize("xd,chunk", [("bf16", 128), ("f32", 128), ("bf16", 100), ("f32", 100)])
def test_single_call_grouped_equals_two_call(xd, chunk):
    wl = inputs.custom(900, 136, 2500, 40, chunk, x_dtype=xd, mask="random:40", tag=960)
    inp = inputs.make_inputs(wl, seed=10)
    d = upload(inp)
    log(f"case single-call grouped {xd} chunk={chunk}")
    loss2, lse2, dH2, dW2 = _run(d, chunk, 3)
    gl = torch.tensor([0.37], dtype=torch.float32, device="cuda")
    one = L.forward_backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], gl, chunk=chunk, dw_chunks=3)
    torch.cuda.synchronize()
    assert float(one["loss"].item()) == loss2 and torch.equal(one["lse"], lse2)
    assert torch.equal(one["dH"], dH2) and torch.equal(one["dW"], dW2)
    ref = oracle.run(inp, g=0.37)
    tol = 1e-5 if xd == "f32" else 1e-2
    assert rel_fro(one["dW"].cpu().numpy(), ref["dW"]) <= tol
    assert rel_fro(one["dH"].cpu().numpy(), ref["dH"]) <= tol
