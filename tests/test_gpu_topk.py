"""GPU tests of the teacher top-K producer (kd_teacher_topk) against the
top-K oracle (oracle/topk.py).

Which K tokens are kept is decided by comparing logits, so both sides must
compare the same values.  Where the logits are exact in fp32 whatever the
summation order (integer-valued inputs with every partial sum below 2^24),
the oracle's fp64 logits equal the kernel's and the records must agree bit
for bit -- ids, order and logits, ties included.  With real-valued inputs the
fp32 accumulation order makes near-equal logits swap, so the test checks
what is unique (each kept logit equals the oracle's logit of that id to fp32
accumulation error, and is at least the oracle's K-th largest minus that
error; every id left out is at most the K-th largest plus that error; the
record is sorted and its ids distinct).
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _run(Hs, Ws, k, chunk, xd):
    H, W = dev(Hs, xd), dev(Ws, xd)
    out = L.teacher_topk(H, W, k=k, chunk=chunk)
    torch.cuda.synchronize()
    return out["ids"].cpu().numpy(), out["logits"].cpu().numpy(), int(out["overflow_rows"].item())


def _unique_integer_logits(n, d, v, seed):
    """z_v = 4096 * (integer dot) + u_v with u_v distinct in [0, 4096): every
    logit of a row distinct, |z| < 2^24, every entry exact in bf16."""
    assert v <= 4096
    rng = np.random.default_rng(seed)
    H = np.zeros((n, d), np.float32)
    W = np.zeros((v, d), np.float32)
    H[:, : d - 3] = 4096.0 * rng.integers(-2, 3, size=(n, d - 3))
    W[:, : d - 3] = rng.integers(-2, 3, size=(v, d - 3))
    u = rng.permutation(4096)[:v]
    H[:, d - 3:] = [256.0, 16.0, 1.0]
    W[:, d - 3] = u // 256
    W[:, d - 2] = (u // 16) % 16
    W[:, d - 1] = u % 16
    return H, W


@pytest.mark.parametrize("xd", ["bf16", "f32"])
@pytest.mark.parametrize("n,d,v,k,chunk", [(300, 64, 3000, 100, 128), (257, 128, 4096, 256, 256), (70, 32, 1500, 1, 64)])
def test_exact_distinct_logits(xd, n, d, v, k, chunk):
    H, W = _unique_integer_logits(n, d, v, seed=n + v)
    Hs = _bf16_bits(H) if xd == "bf16" else H
    Ws = _bf16_bits(W) if xd == "bf16" else W
    log(f"case exact n={n} d={d} v={v} k={k} chunk={chunk} {xd}")
    ids, vals, ovf = _run(Hs, Ws, k, chunk, xd)
    rids, rvals = oracle.teacher_topk(H.astype(np.float64), W.astype(np.float64), k)
    assert ovf == 0
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(vals.astype(np.float64), rvals)


def _unique_integer_logits_wide(n, v, seed):
    """d = 8: z_v = 2^19 (integer dot over 5 entries in [-2, 2]) + u_v with u_v
    distinct in [0, 2^19): every logit of a row distinct, |z| < 2^24, every
    entry exact in bf16 -- for vocabularies up to 2^19."""
    assert v <= 1 << 19
    d = 8
    rng = np.random.default_rng(seed)
    H = np.zeros((n, d), np.float32)
    W = np.zeros((v, d), np.float32)
    H[:, :5] = float(1 << 19) * rng.integers(-2, 3, size=(n, 5))
    W[:, :5] = rng.integers(-2, 3, size=(v, 5))
    u = rng.permutation(1 << 19)[:v]
    H[:, 5:] = [4096.0, 64.0, 1.0]
    W[:, 5] = u // 4096
    W[:, 6] = (u // 64) % 64
    W[:, 7] = u % 64
    return H, W


@pytest.mark.parametrize("v", [200000, 300000, 400000])
def test_exact_distinct_logits_large_vocabulary(v):
    """Every path of the per-row threshold: the sampled maxima of a row held in
    registers (v <= 294912), staged in LDS (v <= 393216), read from memory."""
    n, k, chunk = 64, 100, 64
    H, W = _unique_integer_logits_wide(n, v, seed=v)
    log(f"case exact wide vocabulary n={n} v={v} k={k}")
    ids, vals, ovf = _run(_bf16_bits(H), _bf16_bits(W), k, chunk, "bf16")
    rids, rvals = oracle.teacher_topk(H.astype(np.float64), W.astype(np.float64), k)
    assert ovf == 0
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(vals.astype(np.float64), rvals)


def test_ties_take_lower_ids():
    rng = np.random.default_rng(3)
    n, d, v, k = 200, 8, 3000, 100
    H = rng.integers(-1, 2, size=(n, d)).astype(np.float32)
    W = rng.integers(-1, 2, size=(v, d)).astype(np.float32)
    ids, vals, ovf = _run(_bf16_bits(H), _bf16_bits(W), k, 64, "bf16")
    rids, rvals = oracle.teacher_topk(H.astype(np.float64), W.astype(np.float64), k)
    assert ovf == 0
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(vals.astype(np.float64), rvals)


def test_all_equal_logits():
    n, d, k = 40, 16, 50
    H = np.ones((n, d), np.float32)
    # v within the candidate capacity: exact, ids 0..k-1
    ids, vals, ovf = _run(_bf16_bits(H), _bf16_bits(np.zeros((4000, d), np.float32)), k, 32, "bf16")
    assert ovf == 0
    np.testing.assert_array_equal(ids, np.tile(np.arange(k), (n, 1)))
    assert np.all(vals == 0.0)
    # more tied logits than the capacity: every row is reported
    ids, vals, ovf = _run(_bf16_bits(H), _bf16_bits(np.zeros((9000, d), np.float32)), k, 32, "bf16")
    assert ovf == n
    assert np.all(vals == 0.0) and np.all((ids >= 0) & (ids < 9000))


def _check_valid(ids, vals, H64, W64, rows, k, tol_rel=2e-6):
    Z = H64[rows] @ W64.T
    for r, i in enumerate(rows):
        z = Z[r]
        zk = np.partition(-z, k - 1)[k - 1] * -1.0  # oracle's K-th largest
        tol = tol_rel * (np.abs(H64[i]) @ np.abs(W64).T).max()  # fp32 accumulation error bound scale
        got = ids[r]
        assert len(set(got.tolist())) == k and got.min() >= 0
        assert np.all(np.diff(vals[r]) <= 0)
        assert np.all(np.abs(vals[r] - z[got]) <= tol)
        assert z[got].min() >= zk - 2 * tol
        rest = np.setdiff1d(np.arange(W64.shape[0]), got)
        assert z[rest].max() <= zk + 2 * tol


@pytest.mark.parametrize("n,d,v,k,chunk", [(500, 136, 5000, 100, 200), (300, 64, 777, 256, 128)])
def test_random_inputs_valid(n, d, v, k, chunk):
    wl = inputs.custom(n, d, v, k, chunk, x_dtype="bf16", tag=500 + n)
    inp = inputs.make_inputs(wl, seed=2, only=("H", "W"))
    ids, vals, ovf = _run(inp["H"], inp["W"], k, chunk, "bf16")
    assert ovf == 0
    H64, W64 = oracle.widen(inp["H"], "bf16"), oracle.widen(inp["W"], "bf16")
    _check_valid(ids, vals, H64, W64, np.arange(n), k)
    rids, _ = oracle.teacher_topk(H64, W64, k)
    same = np.mean([len(set(a) & set(b)) / k for a, b in zip(ids.tolist(), rids.tolist())])
    log(f"random inputs: mean overlap with the oracle's record {same:.5f}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_gpt_oss_shape_full_sampled_rows():
    """The whole 32768-row pass at the gpt-oss shapes (H, W standing in for a
    teacher), as bench.py times it: 12 seeded rows in each of the 16 chunks
    checked for validity against the oracle's logits, and the share of ids the
    oracle's record holds as well."""
    wl = inputs.workload("gpt-oss-20b-32k")
    n = wl.n
    inp = inputs.make_inputs(wl, seed=0, n=n, only=("H", "W"))
    log(f"case gpt-oss teacher shape n={n} d={wl.d} v={wl.v} k={wl.k} chunk={wl.chunk}")
    ids, vals, ovf = _run(inp["H"], inp["W"], wl.k, wl.chunk, "bf16")
    assert ovf == 0
    rng = np.random.default_rng([5, 17])
    rows = np.sort(np.concatenate([c * wl.chunk + rng.choice(wl.chunk, 12, replace=False)
                                   for c in range(n // wl.chunk)]))
    H64, W64 = oracle.widen(inp["H"][rows], "bf16"), oracle.widen(inp["W"], "bf16")
    log(f"case gpt-oss teacher shape: oracle on {rows.size} rows across all chunks")
    _check_valid(ids[rows], vals[rows], H64, W64, np.arange(rows.size), wl.k)
    rids, _ = oracle.teacher_topk(H64, W64, wl.k)
    same = np.mean([len(set(a) & set(b)) / wl.k for a, b in zip(ids[rows].tolist(), rids.tolist())])
    log(f"case gpt-oss teacher shape: mean overlap with the oracle's record {same:.5f}")
    assert same >= 0.99
