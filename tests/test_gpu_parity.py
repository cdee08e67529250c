"""GPU parity of the HIP path against the fp64 oracle on small shapes.

Tolerances (written here, applied element by element or per tensor):
  * fp32 inputs: loss relative error <= 1e-5; dH, dW relative Frobenius
    error <= 1e-5; lse relative <= 1e-5;
  * bf16 inputs: loss relative error <= 1e-3; dH, dW relative Frobenius
    error <= 1e-2 (dZ is rounded once to bf16 before the gradient GEMMs);
  * gathered logits: bit-exact where the products are exact (integer-valued
    inputs); otherwise within fp32 accumulation error;
  * chunk size: lse and gathered logits bit-identical across chunk sizes.
The shapes span several projection and dH tiles (256 x 384) and dW tiles
(384 x 256) and end in ragged tails in every dimension.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import dev, log, rel, rel_fro, run_hip, upload

pytestmark = pytest.mark.gpu


def _cmp(inp, out, ref, tol_loss, tol_grad, tol_lse=1e-5, tag=""):
    log(f"[{tag}] loss gpu={out['loss']:.9g} oracle={ref['loss']:.9g}")
    assert rel(out["loss"], ref["loss"]) <= tol_loss, (out["loss"], ref["loss"])
    np.testing.assert_allclose(out["lse"], ref["lse"], rtol=tol_lse, atol=0)
    scale = 1.0 + np.abs(ref["row_loss"])
    assert np.all(np.abs(out["row_loss"] - ref["row_loss"]) <= 10 * tol_loss * scale)
    zscale = 1.0 + np.abs(ref["zg"]).max()
    assert np.abs(out["zg"] - ref["zg"]).max() <= 1e-5 * zscale
    e_dh = rel_fro(out["dH"].cpu().numpy(), ref["dH"])
    e_dw = rel_fro(out["dW"].cpu().numpy(), ref["dW"])
    log(f"[{tag}] rel_fro dH={e_dh:.3g} dW={e_dw:.3g}")
    assert e_dh <= tol_grad and e_dw <= tol_grad


def test_tiny_f32_workload_full():
    wl = inputs.workload("tiny-f32")
    inp = inputs.make_inputs(wl, seed=0)
    log(f"case tiny-f32 n={wl.n} d={wl.d} v={wl.v} k={wl.k} chunk={wl.chunk}")
    out = run_hip(upload(inp), wl.chunk)
    ref = oracle.run(inp)
    _cmp(inp, out, ref, 1e-5, 1e-5, tag="tiny-f32")
    masked = np.nonzero(inp["mask"] == 0)[0]
    assert np.all(out["dH"].cpu().numpy()[masked] == 0.0)
    assert np.all(out["row_loss"][masked] == 0.0)


SMALL = [
    # n, d, v, k, chunk, x_dtype, mask
    (700, 192, 3000, 37, 300, "bf16", "random:50"),
    (513, 136, 1000, 100, 256, "bf16", "tail:40"),
    (300, 64, 520, 16, 300, "f32", "none"),
    (257, 200, 777, 256, 100, "bf16", "none"),
    (1024, 384, 5000, 100, 512, "f32", "random:100"),
    (600, 520, 2000, 64, 256, "bf16", "random:40"),
    # hidden sizes spanning several dW (256-wide) and dH (384-wide) hidden tiles,
    # the last whole or partly filled
    (450, 640, 3001, 50, 200, "f32", "random:30"),
    (333, 960, 2500, 64, 333, "bf16", "none"),
    (260, 1560, 1100, 40, 130, "f32", "tail:20"),
    # the smallest hidden size, and a vocabulary narrower than one wave's 96 columns
    # (three of the four waves of every projection tile hold no column below v)
    (100, 8, 50, 8, 32, "bf16", "random:10"),
    # every vocabulary entry is a teacher id (K = V): the -p terms cover the whole row
    (70, 16, 96, 96, 7, "f32", "none"),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "x".join(map(str, s[:5])) + "-" + s[5])
def test_small_shapes(spec):
    n, d, v, k, chunk, xd, mask = spec
    wl = inputs.custom(n, d, v, k, chunk, x_dtype=xd, mask=mask, tag=200 + n)
    log(f"case {wl.name} chunk={chunk} {xd} mask={mask}")
    inp = inputs.make_inputs(wl, seed=1)
    out = run_hip(upload(inp), chunk, g=0.37)
    ref = oracle.run(inp, g=0.37)
    tl, tg = (1e-5, 1e-5) if xd == "f32" else (1e-3, 1e-2)
    _cmp(inp, out, ref, tl, tg, tag=wl.name)


def _integer_problem(n, d, v, k, seed, dtype):
    rng = np.random.default_rng(seed)
    H = rng.integers(-2, 3, size=(n, d)).astype(np.float32)
    W = rng.integers(-2, 3, size=(v, d)).astype(np.float32)
    ids = np.stack([rng.permutation(v)[:k] for _ in range(n)]).astype(np.int32)
    a = np.round(-np.sort(-3 * rng.standard_normal((n, k)), axis=1)).astype(np.float32)
    if dtype == "bf16":
        Hs, Ws = inputs.f32_to_bf16_bits(H), inputs.f32_to_bf16_bits(W)
        As = inputs.f32_to_bf16_bits(a)
    else:
        Hs, Ws, As = H, W, a
    wl = inputs.custom(n, d, v, k, 64, x_dtype=dtype)
    return {"wl": wl, "n": n, "H": Hs, "W": Ws, "t_ids": ids, "t_logits": As, "mask": None}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_bit_exact_integer_inputs(dtype):
    """Integer-valued H, W in [-2, 2]: every partial sum is an integer below
    2^24, so z is exact in fp32 whatever the order; the gathered logits must
    equal the oracle's bit for bit."""
    inp = _integer_problem(600, 96, 2100, 64, 5, dtype)
    log(f"case integer-exact {dtype}")
    d = upload(inp)
    out = run_hip(d, 128)
    ref = oracle.run(inp)
    assert np.array_equal(out["zg"].astype(np.float64), ref["zg"])


def test_chunk_size_invariance():
    wl = inputs.custom(300, 128, 1500, 20, 64, x_dtype="bf16", mask="random:30", tag=301)
    inp = inputs.make_inputs(wl, seed=2)
    d = upload(inp)
    outs = {}
    for c in (1, 7, 64, 300):
        log(f"case chunk-invariance chunk={c}")
        outs[c] = run_hip(d, c)
    for c in (1, 7, 64):
        assert np.array_equal(outs[c]["lse"], outs[300]["lse"])
        assert np.array_equal(outs[c]["zg"], outs[300]["zg"])
        assert rel(outs[c]["loss"], outs[300]["loss"]) <= 1e-6
        assert torch.equal(outs[c]["dH"], outs[300]["dH"]) or \
            rel_fro(outs[c]["dH"].cpu().numpy(), outs[300]["dH"].cpu().numpy()) <= 1e-6


def test_masked_rows_hold_garbage():
    wl = inputs.custom(400, 64, 900, 30, 128, x_dtype="bf16", mask="random:60", tag=302)
    inp = inputs.make_inputs(wl, seed=3)
    d = upload(inp)
    log("case masked-garbage clean")
    clean = run_hip(d, 128)
    masked = np.nonzero(inp["mask"] == 0)[0]
    ids = inp["t_ids"].copy()
    ids[masked] = -1
    lg = inp["t_logits"].copy()
    lg[masked] = 0x7FC0  # bf16 NaN
    d2 = dict(d)
    d2["t_ids"], d2["t_logits"] = dev(ids), dev(lg, "bf16")
    log("case masked-garbage garbage")
    dirty = run_hip(d2, 128)
    assert dirty["loss"] == clean["loss"]
    assert np.array_equal(dirty["lse"], clean["lse"])
    assert torch.equal(dirty["dH"], clean["dH"]) and torch.equal(dirty["dW"], clean["dW"])
    assert np.all(dirty["dH"].cpu().numpy()[masked] == 0.0)


def test_run_to_run_determinism():
    wl = inputs.custom(600, 256, 4000, 50, 256, x_dtype="bf16", tag=303)
    inp = inputs.make_inputs(wl, seed=4)
    d = upload(inp)
    log("case determinism")
    a, b = run_hip(d, 256), run_hip(d, 256)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["lse"], b["lse"]) and np.array_equal(a["zg"], b["zg"])
    assert torch.equal(a["dH"], b["dH"]) and torch.equal(a["dW"], b["dW"])


def test_dw_accumulates_and_keeps_prior_contents():
    wl = inputs.custom(500, 128, 2000, 40, 200, x_dtype="bf16", tag=304)
    inp = inputs.make_inputs(wl, seed=5)
    d = upload(inp)
    log("case dW accumulation")
    base = run_hip(d, 200)["dW"]
    prior = torch.randn(wl.v, wl.d, device="cuda", dtype=torch.float32)
    once = run_hip(d, 200, dW_init=prior)["dW"]
    # The prior contents enter the fp32 accumulators before a chunk's
    # products, so `once` and `prior + base` round differently: per element
    # about 35 accumulator updates (3 chunks of at most 200 rows, 16 rows per
    # update), each off by at most 2^-24 of a magnitude of a few units.
    torch.testing.assert_close(once, prior + base, rtol=1e-5, atol=1e-5)
    twice = run_hip(d, 200, dW_init=once)["dW"]
    torch.testing.assert_close(twice, prior + 2 * base, rtol=2e-5, atol=2e-5)


def test_g_scales_gradients():
    wl = inputs.custom(300, 64, 700, 10, 128, x_dtype="f32", tag=305)
    inp = inputs.make_inputs(wl, seed=6)
    d = upload(inp)
    log("case g scaling")
    a = run_hip(d, 128, g=1.0)
    b = run_hip(d, 128, g=-2.5)
    # g scales the row coefficient and the teacher term in fp32 before the
    # gradient GEMMs: linear up to fp32 rounding
    assert rel_fro(b["dH"].cpu().numpy(), -2.5 * a["dH"].cpu().numpy()) <= 1e-6
    assert rel_fro(b["dW"].cpu().numpy(), -2.5 * a["dW"].cpu().numpy()) <= 1e-6
    ref = oracle.run(inp, g=-2.5)
    assert rel_fro(b["dH"].cpu().numpy(), ref["dH"]) <= 1e-5
    assert rel_fro(b["dW"].cpu().numpy(), ref["dW"]) <= 1e-5
    z = run_hip(d, 128, g=0.0)
    assert torch.count_nonzero(z["dH"]) == 0 and torch.count_nonzero(z["dW"]) == 0


def test_zero_loss_construction_f32():
    """W = I (D = V = 64), h_i = teacher logits at the K ids and -1e4 elsewhere:
    the student matches the renormalised teacher, so L = 0 up to fp32 rounding."""
    n, k, v = 96, 5, 64
    rng = np.random.default_rng(7)
    ids = np.stack([rng.permutation(v)[:k] for _ in range(n)]).astype(np.int32)
    a = (-np.sort(-3.0 * rng.standard_normal((n, k)), axis=1)).astype(np.float32)
    H = np.full((n, v), -1e4, dtype=np.float32)
    for i in range(n):
        H[i, ids[i]] = a[i]
    inp = {"wl": inputs.custom(n, v, v, k, 32, x_dtype="f32"), "n": n, "H": H,
           "W": np.eye(v, dtype=np.float32), "t_ids": ids, "t_logits": a, "mask": None}
    log("case zero-loss")
    out = run_hip(upload(inp), 32)
    assert abs(out["loss"]) <= 1e-5 * n
    assert out["loss"] >= -1e-5 * n


def test_nonnegative_loss_and_dz_sums():
    """L >= 0 and, because each dZ row sums to 0, the vocabulary sums of dW vanish."""
    wl = inputs.custom(512, 128, 3000, 100, 256, x_dtype="f32", tag=306)
    inp = inputs.make_inputs(wl, seed=8)
    log("case invariants")
    out = run_hip(upload(inp), 256)
    assert out["loss"] >= 0 and np.all(out["row_loss"] >= -1e-5)
    dW = out["dW"].double()
    col = dW.sum(dim=0).abs().max().item()
    assert col <= 1e-5 * dW.abs().sum(dim=0).max().item()


def test_empty_input():
    wl = inputs.custom(0, 64, 500, 8, 32, x_dtype="bf16")
    H = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.randn(500, 64, device="cuda").to(torch.bfloat16)
    ids = torch.empty(0, 8, dtype=torch.int32, device="cuda")
    lg = torch.empty(0, 8, dtype=torch.bfloat16, device="cuda")
    from chunked_kl_loss_row_amd import loss as L
    log("case empty")
    f = L.forward(H, W, ids, lg, None, chunk=32)
    torch.cuda.synchronize()
    assert f["loss"].item() == 0.0
    dW0 = torch.full((500, 64), 3.0, device="cuda")
    dH, dW = L.backward(H, W, ids, lg, None, f["lse"], None, dW=dW0.clone(), chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(dW, dW0)
    del wl


def test_autograd_wrapper():
    wl = inputs.custom(256, 128, 1000, 16, 64, x_dtype="f32", tag=307)
    inp = inputs.make_inputs(wl, seed=9)
    d = upload(inp)
    from chunked_kl_loss_row_amd import loss as L
    h = d["H"].clone().requires_grad_(True)
    w = d["W"].clone().requires_grad_(True)
    log("case autograd")
    lo = L.kd_chunked_kl(h, w, d["t_ids"], d["t_logits"], None, chunk=64)
    (0.5 * lo).backward()
    ref = oracle.run(inp, g=0.5)
    assert rel(lo.item(), ref["loss"]) <= 1e-5
    assert rel_fro(h.grad.cpu().numpy(), ref["dH"]) <= 1e-5
    assert rel_fro(w.grad.cpu().numpy(), ref["dW"]) <= 1e-5


@pytest.mark.parametrize("xd", ["bf16", "f32"])
def test_ids_outside_the_vocabulary_match_nothing(xd):
    """Ids outside [0, v) -- v, v + 1 (padding columns of the last 384-wide
    tile), -1, 2^24 + 5 (id 5 in its low 24 bits) and INT_MIN (0 in its low
    24 bits) -- match no vocabulary entry: gathered logit 0, no -p in dZ, p
    still counted (the oracle's reading for such records).  Both entry points
    against the oracle, and bit for bit with each other."""
    n, d, v, k, chunk = 300, 64, 2001, 16, 128
    wl = inputs.custom(n, d, v, k, chunk, x_dtype=xd, mask="random:20", tag=980)
    inp = inputs.make_inputs(wl, seed=6)
    bad = [v, v + 1, -1, (1 << 24) + 5, -(1 << 31)]
    rows = np.arange(0, n, 7)
    for j, r in enumerate(rows):
        inp["t_ids"][r, j % k] = bad[j % len(bad)]
    inp["mask"][rows] = 1
    log(f"case unmatched ids {xd}: {rows.size} rows")
    d_ = upload(inp)
    out = run_hip(d_, chunk, g=0.37)
    ref = oracle.run(inp, g=0.37)
    tl, tg = (1e-5, 1e-5) if xd == "f32" else (1e-3, 1e-2)
    _cmp(inp, out, ref, tl, tg, tag=f"unmatched-{xd}")
    assert np.all(out["zg"][inp["t_ids"] < 0] == 0.0) and np.all(out["zg"][inp["t_ids"] >= v] == 0.0)
    gl = torch.tensor([0.37], dtype=torch.float32, device="cuda")
    one = L.forward_backward(d_["H"], d_["W"], d_["t_ids"], d_["t_logits"], d_["mask"], gl, chunk=chunk)
    torch.cuda.synchronize()
    assert float(one["loss"].item()) == out["loss"]
    assert torch.equal(one["dH"], out["dH"]) and torch.equal(one["dW"], out["dW"])


@pytest.mark.parametrize("xd", ["f32", "bf16"])
def test_single_entry_vocabulary(xd):
    """V = K = 1: the student and the renormalised teacher are both the point
    mass, so the loss, dZ (Σp·softmax(z) - p = 1 - 1), dH and the dW added are
    0 (the oracle's exactly; the GPU's to fp32 rounding of exp and log near 1:
    a few units in the last place of |z| per row); lse is the single logit."""
    wl = inputs.custom(100, 8, 1, 1, 32, x_dtype=xd, mask="random:10", tag=330)
    inp = inputs.make_inputs(wl, seed=3)
    log(f"case single-entry vocabulary {xd}")
    out = run_hip(upload(inp), 32, g=0.37)
    ref = oracle.run(inp, g=0.37)
    assert ref["loss"] == 0.0 and np.all(ref["row_loss"] == 0.0)
    zmax = float(np.abs(ref["lse"]).max()) + 1.0
    assert np.abs(out["row_loss"]).max() <= 1e-6 * zmax
    assert abs(out["loss"]) <= wl.n * 1e-6 * zmax
    assert out["dH"].abs().max().item() <= 1e-6 and out["dW"].abs().max().item() <= 1e-5
    np.testing.assert_allclose(out["lse"], ref["lse"], rtol=1e-5, atol=0)
