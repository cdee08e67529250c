"""The largest accepted sizes on the GPU, against the oracle.

The host check admits a problem only while every matrix-core tile panel is
addressable with 32-bit byte offsets and every launch stays below 2^32
work-items.  These tests run the path at those limits:

  * the largest vocabulary (v = 4194048 for bf16, 2097024 for fp32: a panel of
    256 padded dZ rows is then just under 2^31 bytes), with teacher ids in the
    last vocabulary tile;
  * the largest chunk (4194296 rows for bf16: a panel of 256 rows of the
    transposed H_c is just under 2^31 bytes, and the H_c transpose takes 65536
    tiles of 64 rows), followed by a ragged chunk;
  * a teacher record of more than 2^26 rows for the validator (2^32 work-items
    at one wave per row).

Rows are checked on seeded samples (the oracle evaluated on exactly those
rows), dW on vocabulary rows summed over all positions from the oracle's own
lse of every row.  Tolerances as in the parity tests: fp32 1e-5, bf16 loss 1e-3 and gradients
1e-2 relative Frobenius; lse 1e-5 relative.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import binding as B
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, oracle_forward_all, rel, rel_fro, upload, vocab_sample

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _fb(d, chunk, g=0.8):
    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=chunk, row_loss=True, zg=True)
    gl = torch.tensor([g], dtype=torch.float32, device="cuda")
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], f["lse"], gl, chunk=chunk,
                        workspace=f["workspace"])
    torch.cuda.synchronize()
    del f["workspace"]
    return f, dH, dW


def _check_rows(f, dH, inp, xd, rows, g, tl, tg, block):
    """lse, row loss, gathered logits and dH on ``rows`` against the oracle
    evaluated on exactly those rows (rows are independent)."""
    H = oracle.widen(inp["H"][rows], xd)
    W = oracle.widen(inp["W"], xd)
    a = oracle.widen(inp["t_logits"][rows], inp["wl"].t_dtype)
    ids = inp["t_ids"][rows]
    m = None if inp["mask"] is None else inp["mask"][rows]
    ref = oracle.kd_forward(H, W, ids, a, m, block=block)
    rt = torch.from_numpy(rows).cuda()
    np.testing.assert_allclose(f["lse"][rt].cpu().numpy(), ref["lse"], rtol=1e-5, atol=0)
    scale = 1.0 + np.abs(ref["row_loss"])
    assert np.all(np.abs(f["row_loss"][rt].cpu().numpy() - ref["row_loss"]) <= 10 * tl * scale)
    zg = f["zg"][rt].cpu().numpy()
    assert np.abs(zg - ref["zg"]).max() <= 1e-5 * (1.0 + np.abs(ref["zg"]).max())
    refb = oracle.kd_backward(H, W, ids, a, m, g=g, want_dw=False, block=block)
    e_dh = rel_fro(dH[rt].cpu().numpy(), refb["dH"])
    log(f"sampled rows: rel_fro dH={e_dh:.3g}")
    assert e_dh <= tg


@pytest.mark.timeout(900)
@pytest.mark.parametrize("xd,v", [("bf16", 4194048), ("f32", 2097024)])
def test_largest_vocabulary(xd, v):
    n, dd, k, chunk, g = 260, 8, 4, 260, 0.8
    x = B.KD_BF16 if xd == "bf16" else B.KD_F32
    assert B.kd_chunked_workspace_size(B.problem(n, dd, v, k, chunk, x)) > 0
    assert B.kd_chunked_workspace_size(B.problem(n, dd, v + 1, k, chunk, x)) == 0
    wl = inputs.custom(n, dd, v, k, chunk, x_dtype=xd, mask="random:13", tag=900 + (xd == "f32"))
    inp = inputs.make_inputs(wl, seed=2)
    # ids in the last (full) vocabulary tile, including v - 1
    inp["t_ids"][::7, 0] = v - 1
    inp["t_ids"][3::7, 1] = v - 200
    assert all(np.unique(inp["t_ids"][r]).size == k for r in range(n))
    log(f"case largest vocabulary {xd} v={v} n={n}")
    f, dH, dW = _fb(upload(inp), chunk, g)
    tl, tg = (1e-5, 1e-5) if xd == "f32" else (1e-3, 1e-2)
    # dH_i sums v products in fp32: each of its 16 k slices adds ~v / 32
    # two-product partial sums (fp32 atom 32x32x2) into one accumulator, a
    # rounding error of about 2^-24 sqrt(v / 32) ~ 1.5e-5 relative for
    # v = 2^21 (2.1e-5 observed).  The fp32 tolerance of 1e-5 is stated for a
    # 4096-entry vocabulary; here the dH tolerance is 1e-4 (dW sums only
    # n = 260 rows and keeps 1e-5).
    tdh = 1e-4 if xd == "f32" else tg
    # sampled rows: both row tiles, the ragged last rows, masked rows
    rows = np.unique(np.concatenate([np.arange(0, n, 13), [1, 2, 255, 256, 257, n - 1],
                                     np.nonzero(inp["mask"] == 0)[0][:3]]))
    log(f"oracle on {rows.size} rows")
    _check_rows(f, dH, inp, xd, rows, g, tl, tdh, block=4)
    # dW rows over all positions: the last vocabulary tile and a seeded sample
    # of the others (half teacher ids), from the oracle's own lse of every row
    voc = np.unique(np.concatenate([np.arange(v - 384, v),
                                    vocab_sample(inp["t_ids"], inp["mask"], v - 384, 256, seed=5)[0]]))
    ref_all = oracle_forward_all(inp, block=4, tag="largest vocabulary")
    ref_u = oracle.dw_vocab_rows(inp["H"], inp["W"], xd, inp["t_ids"], oracle.widen(inp["t_logits"], wl.t_dtype),
                                 inp["mask"], ref_all["lse"], voc, g=g)
    e_dw = rel_fro(dW[torch.from_numpy(voc).cuda()].cpu().numpy(), ref_u)
    col = dW.double().sum(dim=0).abs().max().item()
    log(f"dW on {voc.size} vocabulary rows: rel_fro={e_dw:.3g}; largest column sum {col:.3g}")
    assert e_dw <= tg
    assert col <= 1e-3 * dW.double().abs().sum(dim=0).max().item()


@pytest.mark.timeout(900)
def test_largest_chunk():
    chunk = 4194296
    n, dd, v, k, g = chunk + 1000, 8, 520, 4, 0.8
    assert B.kd_chunked_workspace_size(B.problem(n, dd, v, k, chunk, B.KD_BF16)) > 0
    assert B.kd_chunked_workspace_size(B.problem(n, dd, v, k, chunk + 1, B.KD_BF16)) == 0
    wl = inputs.custom(n, dd, v, k, chunk, x_dtype="bf16", mask="random:5000", tag=910)
    log(f"case largest chunk: generating n={n} chunk={chunk}")
    inp = inputs.make_inputs(wl, seed=2)
    log("case largest chunk: forward + backward on the GPU")
    f, dH, dW = _fb(upload(inp), chunk, g)
    loss = float(f["loss"].item())
    rl = f["row_loss"].cpu().numpy()
    assert loss >= 0.0 and rel(loss, math.fsum(rl.astype(np.float64).tolist())) <= 1e-5
    # sampled rows: spread over the first chunk, its last rows, the ragged second chunk
    rows = np.unique(np.concatenate([inputs.sample_rows(n, 512, seed=4), np.arange(chunk - 3, chunk + 3),
                                     [0, n - 1]]))
    log(f"oracle on {rows.size} rows")
    _check_rows(f, dH, inp, "bf16", rows, g, 1e-3, 1e-2, block=1024)
    e_dh2 = rel_fro(dH[chunk:].cpu().numpy(), oracle.kd_backward(
        oracle.widen(inp["H"][chunk:], "bf16"), oracle.widen(inp["W"], "bf16"), inp["t_ids"][chunk:],
        oracle.widen(inp["t_logits"][chunk:], "bf16"), inp["mask"][chunk:], g=g, want_dw=False)["dH"])
    # the whole dW (every vocabulary row) over all positions, from the oracle's own lse of every row
    ref_all = oracle_forward_all(inp, slice_rows=1 << 20, block=65536, tag="largest chunk")
    assert rel(loss, ref_all["loss"]) <= 1e-3
    log("oracle dW over all rows")
    ref_w = oracle.dw_vocab_rows(inp["H"], inp["W"], "bf16", inp["t_ids"], oracle.widen(inp["t_logits"], "bf16"),
                                 inp["mask"], ref_all["lse"], np.arange(v), g=g, block=65536)
    e_dw = rel_fro(dW.cpu().numpy(), ref_w)
    log(f"second chunk rel_fro dH={e_dh2:.3g}; rel_fro dW={e_dw:.3g}")
    assert e_dh2 <= 1e-2 and e_dw <= 1e-2


@pytest.mark.timeout(600)
def test_validator_beyond_2e26_rows():
    n, k, v = (1 << 26) + 100, 2, 1000
    r = np.arange(n, dtype=np.int64)
    ids = np.empty((n, k), dtype=np.int32)
    ids[:, 0] = r % v
    ids[:, 1] = (r + 1) % v  # two distinct in-range ids per row
    s1, s2 = 1 << 24, (1 << 25) + 7
    ids[3, 1] = ids[3, 0]
    ids[s1, 0] = -1
    ids[s2, 0] = ids[s2, 1]
    ids[n - 1, 1] = v
    # expected from the construction: rows 3 and s2 repeat an id, rows s1 and
    # n - 1 hold an id outside [0, v); the oracle agrees on those rows
    assert oracle.validate_teacher(ids[[3, s1, s2, n - 1]], v) == (2, 2, 1, 0)
    t = torch.from_numpy(ids).cuda()
    log(f"case validator n={n}")
    out = L.validate_teacher(t, v)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [2, 2, s1, 3]
    mask = torch.ones(n, dtype=torch.uint8, device="cuda")
    mask[3] = 0
    mask[n - 1] = 0
    out = L.validate_teacher(t, v, mask)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [1, 1, s1, s2]
