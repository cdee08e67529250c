"""GPU tests of teacher records whose ids repeat within a row.

The cached record holds K distinct ids, but the loss is defined term by term
(one KL term per cached slot), so a repeated id adds its terms: the gathered
logit appears in each of its slots and dZ gets one -p per slot at that
column.  The oracle scatters with np.add.at (pinned for repeats on the CPU).
Planted here:
  * adjacent slots with one id, the first and the last slot with one id,
    one id in three slots, one id in every slot;
  * more than four hits of a row in one 384-wide vocabulary tile (the
    kernels keep up to four per row and tile in LDS; more take the global
    path), with a repeat among them;
  * the last vocabulary entry repeated;
  * random repeats in about a tenth of the rows.
Both entry points (kd_chunked_fwd + kd_chunked_bwd, which recompute the
logits, and kd_chunked_fwd_bwd, which keeps them) are compared with the oracle
-- per planted row as well as per tensor -- and bit for bit with each other.
Tolerances: fp32 1e-5 (loss relative, gradients relative Frobenius), bf16
1e-3 / 1e-2; lse 1e-5 relative.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, rel, rel_fro, upload

pytestmark = pytest.mark.gpu

PLANTED = 7  # rows 0..6 hold the hand-planted patterns


def plant_repeats(ids, v, seed):
    ids = np.array(ids, dtype=np.int32, copy=True)
    n, K = ids.shape
    assert K >= 10 and n >= 64 and v >= 3 * 384
    ids[0, 4] = ids[0, 3]                      # adjacent slots
    ids[1, K - 1] = ids[1, 0]                  # first and last slot
    ids[2, 5] = ids[2, 1]                      # one id in three slots
    ids[2, 9] = ids[2, 1]
    base = 384 * 2                             # six hits in one tile, one of them a repeat
    ids[3, :6] = [base + 0, base + 1, base + 2, base + 3, base + 5, base + 1]
    ids[3, 6:] = np.where((ids[3, 6:] >= base) & (ids[3, 6:] < base + 384), 0, ids[3, 6:])
    ids[4, :] = ids[4, 0]                      # every slot
    ids[5, 2] = v - 1                          # the last vocabulary entry, twice
    ids[5, 7] = v - 1
    ids[6, 0] = ids[6, 1] = ids[6, 2] = 384 * 2 + 7   # a repeated id with two more hits in its tile
    ids[6, 3] = 384 * 2 + 100
    ids[6, 4] = 384 * 2 + 200
    rng = np.random.default_rng([seed, 5])
    rows = rng.choice(np.arange(PLANTED, n), size=max(1, n // 10), replace=False)
    for r in rows:
        a, b = rng.choice(K, size=2, replace=False)
        ids[r, b] = ids[r, a]
    return ids


CASES = [
    # n, d, v, k, chunk, x_dtype, mask, g, tau
    (700, 192, 3000, 37, 300, "bf16", "random:50", 0.37, 1.0),
    (300, 64, 1500, 16, 128, "f32", "none", None, 1.0),
    (513, 136, 1200, 100, 256, "bf16", "tail:40", None, 2.5),
    (257, 128, 1300, 256, 100, "f32", "random:20", -1.5, 0.7),
    (400, 200, 5000, 64, 400, "bf16", "none", None, 1.0),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "x".join(map(str, s[:5])) + f"-{s[5]}-tau{s[8]}")
def test_repeated_ids(spec):
    n, dd, v, k, chunk, xd, mask, g, tau = spec
    wl = inputs.custom(n, dd, v, k, chunk, x_dtype=xd, mask=mask, tag=900 + n)
    inp = inputs.make_inputs(wl, seed=2)
    inp["t_ids"] = plant_repeats(inp["t_ids"], v, seed=n)
    if inp["mask"] is not None:
        inp["mask"][:PLANTED] = 1
    log(f"case repeats {wl.name} chunk={chunk} {xd} mask={mask} g={g} tau={tau}")
    d = upload(inp)
    gl = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda")
    dW0 = torch.randn(v, dd, device="cuda", generator=torch.Generator("cuda").manual_seed(n))

    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=chunk, row_loss=True, zg=True,
                  temperature=tau)
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], f["lse"], gl, dW=dW0.clone(),
                        chunk=chunk, workspace=f["workspace"], temperature=tau)
    s = L.forward_backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], gl, dW=dW0.clone(), chunk=chunk,
                           temperature=tau)
    torch.cuda.synchronize()

    # the two entry points agree bit for bit
    assert torch.equal(s["loss"], f["loss"])
    assert torch.equal(s["lse"], f["lse"])
    assert torch.equal(s["dH"], dH)
    assert torch.equal(s["dW"], dW)

    ref = oracle.run(inp, g=1.0 if g is None else g, tau=tau)
    tol_loss, tol_grad = (1e-5, 1e-5) if xd == "f32" else (1e-3, 1e-2)
    loss = float(f["loss"].item())
    log(f"repeats: loss gpu={loss:.9g} oracle={ref['loss']:.9g}")
    assert rel(loss, ref["loss"]) <= tol_loss
    np.testing.assert_allclose(f["lse"].cpu().numpy(), ref["lse"], rtol=1e-5, atol=0)
    rl = f["row_loss"].cpu().numpy()
    assert np.all(np.abs(rl - ref["row_loss"]) <= 10 * tol_loss * (1.0 + np.abs(ref["row_loss"])))
    zg = f["zg"].cpu().numpy()
    assert np.abs(zg - ref["zg"]).max() <= 1e-5 * (1.0 + np.abs(ref["zg"]).max())
    dH_h = dH.cpu().numpy()
    e_dh = rel_fro(dH_h, ref["dH"])
    e_dw = rel_fro(dW.cpu().numpy() - dW0.cpu().numpy(), ref["dW"])
    log(f"repeats: rel_fro dH={e_dh:.3g} dW={e_dw:.3g}")
    assert e_dh <= tol_grad and e_dw <= tol_grad
    # each planted row on its own: a dropped -p of a repeated id moves that
    # row's dH by about p |w_id|, far above the row's rounding error
    for r in range(PLANTED):
        e = rel_fro(dH_h[r], ref["dH"][r])
        log(f"repeats: planted row {r} rel_fro dH={e:.3g}")
        assert e <= tol_grad, r
