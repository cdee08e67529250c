"""GPU canary tests: nothing is written outside the buffers a call is given.

Every output buffer and the workspace sit between two 4 KiB guard zones
holding a byte pattern; after each call the guards must still hold it, and
the inputs must equal copies taken before the call.  The workspace is handed
over with exactly the size the library asks for.  Shapes are ragged in every
dimension (rows not a multiple of the chunk, vocabulary not a multiple of the
384-wide tiles, hidden size not a multiple of 32, odd K), with masks, for the
forward, the backward (one chunk and two chunks at a time), the single-call
path, the allocation-free forward and the teacher top-K producer.
"""
import pytest
import torch

from chunked_kl_loss_row_amd import binding as B
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import dev, log, upload

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """A device buffer of `count` elements of `dtype` between two guard zones."""

    def __init__(self, count, dtype, fill=None):
        esize = torch.empty(0, dtype=dtype).element_size()
        self.nbytes = count * esize
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype)
        if fill is not None:
            self.t.copy_(fill)

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.raw[:GUARD] == PATTERN).all()) and bool((self.raw[GUARD + self.nbytes:] == PATTERN).all())


SHAPES = [
    # n, d, v, k, chunk, x_dtype, mask
    (517, 136, 2001, 37, 200, "bf16", "random:40"),
    (300, 72, 1000, 7, 128, "f32", "tail:11"),
]


@pytest.mark.parametrize("spec", SHAPES, ids=lambda s: "x".join(map(str, s[:5])) + "-" + s[5])
def test_loss_entry_points_stay_in_bounds(spec):
    n, d, v, k, chunk, xd, mask = spec
    wl = inputs.custom(n, d, v, k, chunk, x_dtype=xd, mask=mask, tag=960 + n)
    inp = inputs.make_inputs(wl, seed=4)
    dd = upload(inp)
    copies = {key: t.clone() for key, t in dd.items() if t is not None}
    H, W, ids, lg, m = dd["H"], dd["W"], dd["t_ids"], dd["t_logits"], dd["mask"]
    for groups in (1, 2):
        prob = L.make_problem(H, W, ids, lg, chunk, 1.0, groups)
        log(f"case canaries {wl.name} chunk={chunk} {xd} dw_chunks={groups}")
        ws = Guarded(B.kd_chunked_workspace_size(prob), torch.uint8)
        loss, lse, rl, zg = Guarded(1, torch.float32), Guarded(n, torch.float32), Guarded(n, torch.float32), \
            Guarded(n * k, torch.float32)
        B.kd_chunked_fwd(prob, H, W, ids, lg, m, loss.t, lse.t, rl.t, zg.t, ws.t)
        assert all(b.intact() for b in (ws, loss, lse, rl, zg))
        g = Guarded(1, torch.float32, torch.tensor([0.5]))
        dH, dW = Guarded(n * d, torch.float32), Guarded(v * d, torch.float32, torch.zeros(v * d))
        B.kd_chunked_bwd(prob, H, W, ids, lg, m, lse.t, g.t, dH.t, dW.t, ws.t)
        assert all(b.intact() for b in (ws, lse, g, dH, dW))
        assert bool(torch.isfinite(dW.t).all()) and bool(torch.isfinite(dH.t).all())
        # the single-call path
        wsf = Guarded(B.kd_chunked_fwd_bwd_workspace_size(prob), torch.uint8)
        loss2, lse2 = Guarded(1, torch.float32), Guarded(n, torch.float32)
        dH2, dW2 = Guarded(n * d, torch.float32), Guarded(v * d, torch.float32, torch.zeros(v * d))
        B.kd_chunked_fwd_bwd(prob, H, W, ids, lg, m, g.t, loss2.t, lse2.t, dH2.t, dW2.t, wsf.t)
        assert all(b.intact() for b in (wsf, loss2, lse2, dH2, dW2, g))
        assert torch.equal(dH2.t, dH.t) and torch.equal(dW2.t, dW.t) and torch.equal(lse2.t, lse.t)
    # the allocation-free forward (its scratch is the library's own)
    prob = L.make_problem(H, W, ids, lg, chunk)
    loss3, lse3, rl3, zg3 = Guarded(1, torch.float32), Guarded(n, torch.float32), Guarded(n, torch.float32), \
        Guarded(n * k, torch.float32)
    B.kd_chunked_fwd_noalloc(prob, H, W, ids, lg, m, loss3.t, lse3.t, rl3.t, zg3.t)
    assert all(b.intact() for b in (loss3, lse3, rl3, zg3))
    assert torch.equal(lse3.t, lse.t) and torch.equal(zg3.t, zg.t)
    torch.cuda.synchronize()
    for key, t in copies.items():
        assert torch.equal(dd[key], t), key


@pytest.mark.parametrize("xd", ["bf16", "f32"])
def test_teacher_topk_stays_in_bounds(xd):
    n, d, v, k, chunk = 333, 72, 2001, 37, 128
    wl = inputs.custom(n, d, v, k, chunk, x_dtype=xd, tag=970)
    inp = inputs.make_inputs(wl, seed=5, only=("H", "W"))
    Hd, Wd = dev(inp["H"], xd), dev(inp["W"], xd)
    cH, cW = Hd.clone(), Wd.clone()
    prob = B.problem(n, d, v, k, chunk, B.KD_BF16 if xd == "bf16" else B.KD_F32)
    log(f"case canaries top-K {xd}")
    ws = Guarded(B.kd_teacher_topk_workspace_size(prob), torch.uint8)
    ids, lg, ovf = Guarded(n * k, torch.int32), Guarded(n * k, torch.float32), Guarded(1, torch.int32)
    B.kd_teacher_topk(prob, Hd, Wd, ids.t, lg.t, ovf.t, ws.t)
    assert all(b.intact() for b in (ws, ids, lg, ovf))
    assert int(ovf.t.item()) == 0
    got = ids.t.view(n, k).cpu().numpy()
    assert got.min() >= 0 and got.max() < v
    assert torch.equal(Hd, cH) and torch.equal(Wd, cW)
