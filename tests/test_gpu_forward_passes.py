"""GPU tests of the forward's multi-chunk passes.

kd_chunked_fwd keeps no dZ, so it runs up to 8 chunks per pass when the
workspace (sized for the backward's chunk of dZ) has room.  Every row's lse,
gathered logits and row loss are computed the same way whatever the pass,
and the running loss adds chunk-sized slices in order.  So, on shapes that
take several passes with a ragged last one (the vocabulary is wide enough
that 8 chunks of forward state fit in one chunk of dZ):
  * loss and lse equal kd_chunked_fwd_bwd's (one chunk at a time) bit for bit;
  * lse, gathered logits and row losses equal those of a single pass over all
    rows bit for bit, the loss (other slices) to 1e-6 relative;
  * all of them match the fp64 oracle at the parity tolerances (loss 1e-3 in
    bf16, 1e-5 in fp32; lse 1e-5 relative; gathered logits 1e-5 of the
    largest).
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log, rel, upload

pytestmark = pytest.mark.gpu

CASES = [
    # n, d, v, k, chunk, x_dtype, mask
    (5000, 136, 20000, 40, 200, "bf16", "random:300"),  # 8-chunk passes of 1600 rows, last one 200
    (3333, 64, 2000, 16, 100, "f32", "tail:50"),         # passes of 800 rows, last one 133
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "x".join(map(str, s[:5])) + "-" + s[5])
def test_forward_passes(spec):
    n, dd, v, k, chunk, xd, mask = spec
    wl = inputs.custom(n, dd, v, k, chunk, x_dtype=xd, mask=mask, tag=600 + n)
    log(f"case forward passes {wl.name} chunk={chunk} {xd} mask={mask}")
    inp = inputs.make_inputs(wl, seed=5)
    d = upload(inp)
    fp = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=chunk, row_loss=True, zg=True)
    one = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], chunk=n, row_loss=True, zg=True)
    fb = L.forward_backward(d["H"], d["W"], d["t_ids"], d["t_logits"], d["mask"], None, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(fp["loss"], fb["loss"])
    assert torch.equal(fp["lse"], fb["lse"])
    for key in ("lse", "zg", "row_loss"):
        assert torch.equal(fp[key], one[key]), key
    assert rel(float(fp["loss"].item()), float(one["loss"].item())) <= 1e-6

    x = oracle.widen_inputs(inp)
    ref = oracle.kd_forward(x["H"], x["W"], x["t_ids"], x["t_logits"], x["mask"])
    loss = float(fp["loss"].item())
    log(f"[{wl.name}] loss gpu={loss:.9g} oracle={ref['loss']:.9g}")
    assert rel(loss, ref["loss"]) <= (1e-3 if xd == "bf16" else 1e-5)
    np.testing.assert_allclose(fp["lse"].cpu().numpy(), ref["lse"], rtol=1e-5, atol=0)
    zg = fp["zg"].cpu().numpy()
    assert np.abs(zg - ref["zg"]).max() <= 1e-5 * (1.0 + np.abs(ref["zg"]).max())
    masked = np.nonzero(inp["mask"] == 0)[0]
    assert masked.size > 0 and np.all(fp["row_loss"].cpu().numpy()[masked] == 0.0)
