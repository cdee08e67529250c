"""Full-size workloads on the GPU, checked against the oracle on seeded subsets.

Each workload runs forward + backward over all N positions with its own chunk
size (the launch configuration bench.py times).  The fp64 oracle cannot
afford N x V logits at these sizes, so the checks are:
  * sampled rows S (512 seeded positions): lse, row loss, gathered logits and
    dH rows against the oracle evaluated on exactly those rows;
  * sampled vocabulary rows U (256 ids: half drawn from the teacher ids of
    unmasked rows, half uniform over the vocabulary) of the full run's dW,
    which sums over ALL N positions: the oracle forms those dZ columns from
    the GPU's lse (already checked on S);
  * a second run with the mask restricted to S: the loss and the WHOLE dW
    (every vocab row) then come from S alone, which the oracle computes;
  * properties that hold at any size: loss = sum of row losses, L >= 0, the
    vocabulary sums of dW vanish (each dZ row sums to zero).
Tolerances: loss relative <= 1e-3, gradients relative Frobenius <= 1e-2
(bf16 inputs), lse relative <= 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, rel, rel_fro, upload, vocab_sample

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

S_ROWS = 512
U_IDS = 256



@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["llama3.2-3b-8k", "gpt-oss-20b-32k", "gpt-oss-120b-b4x32k", "long-256k"])
def test_full_workload_sampled(name):
    wl = inputs.workload(name)
    log(f"case {name}: generating n={wl.n} d={wl.d} v={wl.v} k={wl.k} chunk={wl.chunk}")
    inp = inputs.make_inputs(wl, seed=0)
    d = upload(inp)
    log(f"case {name}: full forward + backward on the GPU")
    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=wl.chunk, row_loss=True,
                  zg=True)
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], f["lse"], None,
                        chunk=wl.chunk, workspace=f["workspace"])
    torch.cuda.synchronize()
    loss = float(f["loss"].item())
    rows = inputs.sample_rows(wl.n, S_ROWS, seed=0)
    rows_t = torch.from_numpy(rows).cuda()
    lse = f["lse"][rows_t].cpu().numpy()
    rl_all = f["row_loss"].cpu().numpy()
    zg = f["zg"][rows_t].cpu().numpy()
    dH_s = dH[rows_t].cpu().numpy()

    # size-independent properties
    assert loss >= 0.0
    assert rel(loss, math.fsum(rl_all.astype(np.float64).tolist())) <= 1e-5
    col = dW.double().sum(dim=0).abs().max().item()
    assert col <= 1e-3 * dW.double().abs().sum(dim=0).max().item()
    voc, hit = vocab_sample(inp["t_ids"], inp["mask"], wl.v, U_IDS)
    dW_u = dW[torch.from_numpy(voc).cuda()].cpu().numpy()
    lse_all = f["lse"].cpu().numpy()
    del dH, dW

    log(f"case {name}: oracle dW on {voc.size} vocab rows over all {wl.n} positions")
    ref_u = oracle.dw_vocab_rows(inp["H"], inp["W"], wl.x_dtype, inp["t_ids"],
                                 oracle.widen(inp["t_logits"], wl.t_dtype), inp["mask"], lse_all, voc)
    is_hit = np.isin(voc, hit)
    e_hit = rel_fro(dW_u[is_hit], ref_u[is_hit])
    e_uni = rel_fro(dW_u[~is_hit], ref_u[~is_hit])
    log(f"case {name}: full-run dW vocab rows rel_fro hit={e_hit:.3g} uniform={e_uni:.3g}")
    assert e_hit <= 1e-2 and e_uni <= 1e-2

    log(f"case {name}: oracle on {rows.size} sampled rows")
    # the oracle sees exactly the sampled positions (rows are independent)
    Hs = oracle.widen(inp["H"][rows], wl.x_dtype)
    Wx = oracle.widen(inp["W"], wl.x_dtype)
    ids_s = inp["t_ids"][rows]
    lg_s = oracle.widen(inp["t_logits"][rows], wl.t_dtype)
    m_s = None if inp["mask"] is None else inp["mask"][rows]
    ref_f = oracle.kd_forward(Hs, Wx, ids_s, lg_s, m_s)
    np.testing.assert_allclose(lse, ref_f["lse"], rtol=1e-5, atol=0)
    scale = 1.0 + np.abs(ref_f["row_loss"])
    assert np.all(np.abs(rl_all[rows] - ref_f["row_loss"]) <= 1e-3 * scale)
    assert np.abs(zg - ref_f["zg"]).max() <= 1e-4 * (1.0 + np.abs(ref_f["zg"]).max())
    ref_b = oracle.kd_backward(Hs, Wx, ids_s, lg_s, m_s, want_dw=True)
    e_dh = rel_fro(dH_s, ref_b["dH"])
    log(f"case {name}: sampled rows rel_fro dH={e_dh:.3g}")
    assert e_dh <= 1e-2

    # masked-subset run: the whole dW and the loss come from the sampled rows
    sub = np.zeros(wl.n, dtype=np.uint8)
    sub[rows] = 1
    if inp["mask"] is not None:
        sub &= inp["mask"]
    sub_t = torch.from_numpy(sub).cuda()
    log(f"case {name}: masked-subset run")
    f2 = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], sub_t, chunk=wl.chunk,
                   workspace=f["workspace"])
    dH2, dW2 = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], sub_t, f2["lse"], None,
                          chunk=wl.chunk, workspace=f["workspace"])
    torch.cuda.synchronize()
    loss2 = float(f2["loss"].item())
    ref_loss2 = math.fsum(ref_f["row_loss"][sub[rows] != 0].tolist())
    log(f"case {name}: subset loss gpu={loss2:.9g} oracle={ref_loss2:.9g}")
    assert rel(loss2, ref_loss2) <= 1e-3
    nz_rows = torch.nonzero(dH2.abs().sum(dim=1)).flatten().cpu().numpy()
    assert set(nz_rows.tolist()) <= set(rows.tolist())
    e_dw = rel_fro(dW2.cpu().numpy(), ref_b["dW"])
    log(f"case {name}: masked-subset rel_fro dW={e_dw:.3g}")
    assert e_dw <= 1e-2


@pytest.mark.timeout(600)
def test_single_call_full_size_bitwise():
    """kd_chunked_fwd_bwd at the 32K gpt-oss workload equals kd_chunked_fwd +
    kd_chunked_bwd bit for bit (same fp32 logits, same dZ formula)."""
    wl = inputs.workload("gpt-oss-20b-32k")
    log(f"case single-call {wl.name}: generating")
    inp = inputs.make_inputs(wl, seed=1)
    d = upload(inp)
    log("case single-call: two calls")
    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=wl.chunk)
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], f["lse"], None, chunk=wl.chunk,
                        workspace=f["workspace"])
    torch.cuda.synchronize()
    del f["workspace"]
    log("case single-call: one call")
    g = L.forward_backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], None, chunk=wl.chunk)
    torch.cuda.synchronize()
    assert torch.equal(g["loss"], f["loss"])
    assert torch.equal(g["lse"], f["lse"])
    assert torch.equal(g["dH"], dH)
    assert torch.equal(g["dW"], dW)
