"""Full-size workloads on the GPU, checked against the oracle.

Each workload runs forward + backward over all N positions with its own chunk
size and the backward in groups of two chunks (dw_chunks = 2), the launch
configuration bench.py times.  No oracle call ever receives a value the GPU
computed:
  * llama3.2-3b-8k (8192 rows): the whole problem against the oracle -- every
    row's lse, row loss, gathered logits and dH, the loss and the whole dW;
  * gpt-oss-20b-32k (32768 rows): the oracle's forward over all rows (lse, row
    loss, gathered logits, the full-N loss); dH on 512 seeded rows; 256
    vocabulary rows of the full run's dW (a sum over ALL positions), which the
    oracle forms from its own lse; and a second run with the mask restricted
    to the sampled rows (the loss and the WHOLE dW then come from those rows);
  * gpt-oss-120b-b4x32k and long-256k (131072 / 262144 rows, beyond what the
    oracle's forward over every row costs here): 512 seeded rows (lse, row
    loss, gathered logits, dH) and the masked-subset run;
  * every workload: properties that hold at any size (loss = sum of row
    losses, L >= 0, the vocabulary sums of dW vanish).
Tolerances: loss relative <= 1e-3, gradients relative Frobenius <= 1e-2
(bf16 inputs), lse relative <= 1e-5; gathered logits within fp32
accumulation error.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, oracle_forward_all, rel, rel_fro, upload, vocab_sample

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

S_ROWS = 512
U_IDS = 256


# the launch configuration bench.py times: the backward takes two chunks at once
DW_CHUNKS = 2


def _full_run(d, wl, mask=None, workspace=None, row_loss=True, zg=True):
    m = d["mask"] if mask is None else mask
    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], m, chunk=wl.chunk, row_loss=row_loss, zg=zg,
                  workspace=workspace, dw_chunks=DW_CHUNKS)
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], m, f["lse"], None, chunk=wl.chunk,
                        workspace=f["workspace"], dw_chunks=DW_CHUNKS)
    torch.cuda.synchronize()
    return f, dH, dW


def _invariants(f, dW):
    loss = float(f["loss"].item())
    rl = f["row_loss"].cpu().numpy()
    assert loss >= 0.0
    assert rel(loss, math.fsum(rl.astype(np.float64).tolist())) <= 1e-5
    col = dW.double().sum(dim=0).abs().max().item()
    assert col <= 1e-3 * dW.double().abs().sum(dim=0).max().item()
    return loss, rl


def _sampled_rows(name, inp, wl, f, dH, rows):
    """lse, row loss, gathered logits and dH of the sampled rows against the
    oracle evaluated on exactly those rows (rows are independent)."""
    rows_t = torch.from_numpy(rows).cuda()
    log(f"case {name}: oracle on {rows.size} sampled rows")
    Hs = oracle.widen(inp["H"][rows], wl.x_dtype)
    Wx = oracle.widen(inp["W"], wl.x_dtype)
    ids_s = inp["t_ids"][rows]
    lg_s = oracle.widen(inp["t_logits"][rows], wl.t_dtype)
    m_s = None if inp["mask"] is None else inp["mask"][rows]
    ref_f = oracle.kd_forward(Hs, Wx, ids_s, lg_s, m_s)
    np.testing.assert_allclose(f["lse"][rows_t].cpu().numpy(), ref_f["lse"], rtol=1e-5, atol=0)
    scale = 1.0 + np.abs(ref_f["row_loss"])
    assert np.all(np.abs(f["row_loss"][rows_t].cpu().numpy() - ref_f["row_loss"]) <= 1e-3 * scale)
    zg = f["zg"][rows_t].cpu().numpy()
    assert np.abs(zg - ref_f["zg"]).max() <= 1e-4 * (1.0 + np.abs(ref_f["zg"]).max())
    ref_b = oracle.kd_backward(Hs, Wx, ids_s, lg_s, m_s, want_dw=True)
    e_dh = rel_fro(dH[rows_t].cpu().numpy(), ref_b["dH"])
    log(f"case {name}: sampled rows rel_fro dH={e_dh:.3g}")
    assert e_dh <= 1e-2
    return ref_f, ref_b


def _masked_subset(name, inp, wl, d, f, rows, ref_f, ref_b):
    """A second run with the mask restricted to the sampled rows: the loss and
    the whole dW come from those rows alone, which the oracle computes."""
    sub = np.zeros(wl.n, dtype=np.uint8)
    sub[rows] = 1
    if inp["mask"] is not None:
        sub &= inp["mask"]
    log(f"case {name}: masked-subset run")
    f2, dH2, dW2 = _full_run(d, wl, mask=torch.from_numpy(sub).cuda(), workspace=f["workspace"], row_loss=False,
                             zg=False)
    loss2 = float(f2["loss"].item())
    ref_loss2 = math.fsum(ref_f["row_loss"][sub[rows] != 0].tolist())
    log(f"case {name}: subset loss gpu={loss2:.9g} oracle={ref_loss2:.9g}")
    assert rel(loss2, ref_loss2) <= 1e-3
    nz_rows = torch.nonzero(dH2.abs().sum(dim=1)).flatten().cpu().numpy()
    assert set(nz_rows.tolist()) <= set(rows.tolist())
    e_dw = rel_fro(dW2.cpu().numpy(), ref_b["dW"])
    log(f"case {name}: masked-subset rel_fro dW={e_dw:.3g}")
    assert e_dw <= 1e-2


@pytest.mark.timeout(900)
def test_llama_8k_full_against_oracle():
    wl = inputs.workload("llama3.2-3b-8k")
    log(f"case {wl.name}: generating n={wl.n} d={wl.d} v={wl.v} k={wl.k} chunk={wl.chunk}")
    inp = inputs.make_inputs(wl, seed=0)
    d = upload(inp)
    log(f"case {wl.name}: full forward + backward on the GPU")
    f, dH, dW = _full_run(d, wl)
    loss, rl = _invariants(f, dW)
    lse, zg = f["lse"].cpu().numpy(), f["zg"].cpu().numpy()
    dH, dW = dH.cpu().numpy(), dW.cpu().numpy()
    # the oracle over every row, in slices (rows are independent; dW sums the slices)
    Wx = oracle.widen(inp["W"], wl.x_dtype)
    ref_dW = np.zeros((wl.v, wl.d))
    ref_dH = np.empty((wl.n, wl.d))
    ref_lse, ref_rl, ref_zg = np.empty(wl.n), np.empty(wl.n), np.empty((wl.n, wl.k))
    for r0 in range(0, wl.n, 1024):
        r1 = min(wl.n, r0 + 1024)
        Hs = oracle.widen(inp["H"][r0:r1], wl.x_dtype)
        lg = oracle.widen(inp["t_logits"][r0:r1], wl.t_dtype)
        rf = oracle.kd_forward(Hs, Wx, inp["t_ids"][r0:r1], lg, None)
        rb = oracle.kd_backward(Hs, Wx, inp["t_ids"][r0:r1], lg, None, want_dw=True)
        ref_lse[r0:r1], ref_rl[r0:r1], ref_zg[r0:r1] = rf["lse"], rf["row_loss"], rf["zg"]
        ref_dH[r0:r1] = rb["dH"]
        ref_dW += rb["dW"]
        log(f"case {wl.name}: oracle rows {r1}/{wl.n}")
    ref_loss = math.fsum(ref_rl.tolist())
    log(f"case {wl.name}: loss gpu={loss:.9g} oracle={ref_loss:.9g}")
    assert rel(loss, ref_loss) <= 1e-3
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-5, atol=0)
    assert np.all(np.abs(rl - ref_rl) <= 1e-3 * (1.0 + np.abs(ref_rl)))
    assert np.abs(zg - ref_zg).max() <= 1e-4 * (1.0 + np.abs(ref_zg).max())
    e_dh, e_dw = rel_fro(dH, ref_dH), rel_fro(dW, ref_dW)
    log(f"case {wl.name}: rel_fro dH={e_dh:.3g} dW={e_dw:.3g}")
    assert e_dh <= 1e-2 and e_dw <= 1e-2


@pytest.mark.timeout(1200)
def test_gpt_oss_32k_full_forward_against_oracle():
    wl = inputs.workload("gpt-oss-20b-32k")
    name = wl.name
    log(f"case {name}: generating n={wl.n} d={wl.d} v={wl.v} k={wl.k} chunk={wl.chunk}")
    inp = inputs.make_inputs(wl, seed=0)
    d = upload(inp)
    log(f"case {name}: full forward + backward on the GPU")
    f, dH, dW = _full_run(d, wl)
    loss, rl = _invariants(f, dW)
    voc, hit = vocab_sample(inp["t_ids"], inp["mask"], wl.v, U_IDS)
    dW_u = dW[torch.from_numpy(voc).cuda()].cpu().numpy()
    rows = inputs.sample_rows(wl.n, S_ROWS, seed=0)
    ref_f, ref_b = _sampled_rows(name, inp, wl, f, dH, rows)
    del dH, dW
    # the oracle's forward over every row: the full-N loss, every row's lse,
    # row loss and gathered logits
    ref = oracle_forward_all(inp, tag=name)
    log(f"case {name}: loss gpu={loss:.9g} oracle={ref['loss']:.9g}")
    assert rel(loss, ref["loss"]) <= 1e-3
    np.testing.assert_allclose(f["lse"].cpu().numpy(), ref["lse"], rtol=1e-5, atol=0)
    assert np.all(np.abs(rl - ref["row_loss"]) <= 1e-3 * (1.0 + np.abs(ref["row_loss"])))
    zg = f["zg"].cpu().numpy()
    assert np.abs(zg - ref["zg"]).max() <= 1e-4 * (1.0 + np.abs(ref["zg"]).max())
    # vocabulary rows of the full run's dW (sums over all positions), from the oracle's own lse
    log(f"case {name}: oracle dW on {voc.size} vocab rows over all {wl.n} positions")
    ref_u = oracle.dw_vocab_rows(inp["H"], inp["W"], wl.x_dtype, inp["t_ids"],
                                 oracle.widen(inp["t_logits"], wl.t_dtype), inp["mask"], ref["lse"], voc)
    is_hit = np.isin(voc, hit)
    e_hit = rel_fro(dW_u[is_hit], ref_u[is_hit])
    e_uni = rel_fro(dW_u[~is_hit], ref_u[~is_hit])
    log(f"case {name}: full-run dW vocab rows rel_fro hit={e_hit:.3g} uniform={e_uni:.3g}")
    assert e_hit <= 1e-2 and e_uni <= 1e-2
    _masked_subset(name, inp, wl, d, f, rows, ref_f, ref_b)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["gpt-oss-120b-b4x32k", "long-256k"])
def test_large_workload_sampled(name):
    wl = inputs.workload(name)
    log(f"case {name}: generating n={wl.n} d={wl.d} v={wl.v} k={wl.k} chunk={wl.chunk}")
    inp = inputs.make_inputs(wl, seed=0)
    d = upload(inp)
    log(f"case {name}: full forward + backward on the GPU")
    f, dH, dW = _full_run(d, wl)
    _invariants(f, dW)
    del dW
    rows = inputs.sample_rows(wl.n, S_ROWS, seed=0)
    ref_f, ref_b = _sampled_rows(name, inp, wl, f, dH, rows)
    del dH
    _masked_subset(name, inp, wl, d, f, rows, ref_f, ref_b)


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
