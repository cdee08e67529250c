"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: 50-digit mpmath loops over the definition (stored fixture and
  live recomputation), including masked rows, K = 1 and K = V;
* gradients: 50-digit central differences of the brute-force loss;
* closed forms: K = 1, equal teacher logits, W = 0, uniform teacher with W = 0,
  the zero-loss construction;
* invariants: L >= 0, dZ rows sum to 0, dW column sums vanish, masked rows,
  shift invariances, g-linearity, K-permutation;
* library routines: scipy.special.logsumexp / softmax / rel_entr and torch
  CPU fp64 autograd of log_softmax + gather + kl_div.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special as sps

import oracle
from oracle import bruteforce
from oracle_cases import TINY, case_problem, tiny_problem

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    cases = []
    for name in ("tiny_bruteforce.json", "tiny_bruteforce_tau.json"):
        with open(os.path.join(HERE, "golden", name)) as f:
            cases += json.load(f)["cases"]
    return cases


def _arr(x):
    return np.array([[float(mpmath.mpf(v)) for v in r] for r in x])


def rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_golden_bruteforce_forward(case):
    H, W = np.array(case["H"]), np.array(case["W"])
    ids, a = np.array(case["t_ids"]), np.array(case["t_logits"])
    mask = None
    if case["masked"]:
        mask = np.ones(case["n"], np.uint8)
        mask[case["masked"]] = 0
    f = oracle.kd_forward(H, W, ids, a, mask, tau=case.get("tau", 1.0))
    assert abs(f["loss"] - float(mpmath.mpf(case["loss"]))) <= 1e-13 * abs(float(mpmath.mpf(case["loss"])))
    np.testing.assert_allclose(f["lse"], [float(mpmath.mpf(x)) for x in case["lse"]], rtol=1e-14)
    np.testing.assert_allclose(f["row_loss"], [float(mpmath.mpf(x)) for x in case["row_loss"]],
                               rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_golden_bruteforce_gradient(case):
    H, W = np.array(case["H"]), np.array(case["W"])
    ids, a = np.array(case["t_ids"]), np.array(case["t_logits"])
    mask = None
    if case["masked"]:
        mask = np.ones(case["n"], np.uint8)
        mask[case["masked"]] = 0
    b = oracle.kd_backward(H, W, ids, a, mask, g=case["g"], tau=case.get("tau", 1.0))
    assert rel(b["dH"], _arr(case["dH"])) <= 1e-12
    assert rel(b["dW"], _arr(case["dW"])) <= 1e-12


def test_golden_fixture_regenerates():
    """The stored brute-force values are what the brute force computes now."""
    case = _golden()[0]
    L, _, _ = bruteforce.loss(case["H"], case["W"], case["t_ids"], case["t_logits"],
                              [0 if i in case["masked"] else 1 for i in range(case["n"])])
    with mpmath.workdps(50):
        assert mpmath.almosteq(L, mpmath.mpf(case["loss"]), rel_eps=mpmath.mpf("1e-25"))


@pytest.mark.parametrize("spec", TINY, ids=lambda s: s[0])
def test_bruteforce_live(spec):
    H, W, ids, a, mask = case_problem(spec, seed_offset=1000, w_scale=2.5, logit_scale=5.0)
    L, lses, rls = bruteforce.loss(H.tolist(), W.tolist(), ids.tolist(), a.tolist(),
                                   None if mask is None else mask.tolist())
    f = oracle.kd_forward(H, W, ids, a, mask)
    assert abs(f["loss"] - float(L)) <= 1e-12 * abs(float(L))
    np.testing.assert_allclose(f["lse"], [float(x) for x in lses], rtol=1e-14)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_teacher_k1_is_point_mass():
    p, negent, s = oracle.teacher_distribution(np.array([[3.7], [-120.0]]))
    assert np.all(p == 1.0) and np.all(negent == 0.0) and np.all(s == 1.0)


def test_teacher_equal_logits_uniform():
    for K in (2, 16, 100, 256):
        p, negent, s = oracle.teacher_distribution(np.full((3, K), 1.25))
        np.testing.assert_allclose(p, 1.0 / K, rtol=1e-15)
        np.testing.assert_allclose(negent, -math.log(K), rtol=1e-14)
        np.testing.assert_allclose(s, 1.0, rtol=1e-14)


def test_teacher_matches_scipy_softmax_and_shift():
    rng = np.random.default_rng(0)
    a = 3.0 * rng.standard_normal((50, 100))
    p, negent, _ = oracle.teacher_distribution(a)
    np.testing.assert_allclose(p, sps.softmax(a, axis=1), rtol=1e-13)
    p2, negent2, _ = oracle.teacher_distribution(a + 123.456)
    np.testing.assert_allclose(p2, p, rtol=1e-11)
    np.testing.assert_allclose(negent2, negent, rtol=1e-11)


def test_teacher_neg_inf_entries():
    p, negent, s = oracle.teacher_distribution(np.array([[0.0, -np.inf, 0.0]]))
    np.testing.assert_allclose(p, [[0.5, 0.0, 0.5]])
    np.testing.assert_allclose(negent, [-math.log(2)])


def test_zero_weights_lse_is_log_v():
    n, d, v, k = 5, 8, 300, 7
    H, _, ids, a, _ = tiny_problem(n, d, v, k, 3)
    f = oracle.kd_forward(H, np.zeros((v, d)), ids, a)
    np.testing.assert_allclose(f["lse"], math.log(v), rtol=1e-15)


def test_uniform_teacher_zero_weights_closed_form():
    """W = 0 and equal teacher logits: every row costs log(V / K)."""
    n, d, v, k = 256, 128, 4096, 16
    rng = np.random.default_rng(1)
    H = rng.standard_normal((n, d))
    ids = np.stack([rng.permutation(v)[:k] for _ in range(n)])
    f = oracle.kd_forward(H, np.zeros((v, d)), ids, np.zeros((n, k)))
    np.testing.assert_allclose(f["row_loss"], math.log(256.0), rtol=1e-14)
    assert abs(f["loss"] - n * 5.545177444479562) <= 1e-12 * n * 5.545


def _zero_loss_problem(n=6, k=5):
    """D = V = 64, W = I, h_i[v] = teacher logit at v = t_ik, -1e4 elsewhere:
    the student equals the renormalised teacher on the K ids and puts no mass
    elsewhere, so every row's KL is 0."""
    v = d = 64
    rng = np.random.default_rng(7)
    ids = np.stack([rng.permutation(v)[:k] for _ in range(n)])
    a = -np.sort(-3.0 * rng.standard_normal((n, k)), axis=1)
    H = np.full((n, d), -1e4)
    for i in range(n):
        H[i, ids[i]] = a[i]
    return H, np.eye(v), ids, a


def test_zero_loss_construction():
    H, W, ids, a = _zero_loss_problem()
    f = oracle.kd_forward(H, W, ids, a)
    assert abs(f["loss"]) <= 1e-12
    b = oracle.kd_backward(H, W, ids, a)
    # dZ is zero up to fp64 rounding (~1e-16); dW = dZ^T H multiplies that by
    # the 1e4-sized entries of H, so its bound is 1e4 times looser.
    assert np.abs(b["dH"]).max() <= 1e-12 and np.abs(b["dW"]).max() <= 1e-8


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def _rand_problem(seed=5, n=40, d=24, v=97, k=10, masked=(3, 17)):
    return tiny_problem(n, d, v, k, seed, masked, w_scale=1.0, logit_scale=3.0)


def test_loss_nonnegative():
    for seed in range(6):
        H, W, ids, a, mask = _rand_problem(seed)
        f = oracle.kd_forward(H, W, ids, a, mask)
        assert f["loss"] >= 0.0 and np.all(f["row_loss"] >= -1e-12)


def test_dz_rows_sum_to_zero_and_masked_rows():
    H, W, ids, a, mask = _rand_problem()
    b = oracle.kd_backward(H, W, ids, a, mask, want_dz=True)
    np.testing.assert_allclose(b["dZ"].sum(axis=1), 0.0, atol=1e-14)
    masked = np.nonzero(mask == 0)[0]
    assert np.all(b["dZ"][masked] == 0.0) and np.all(b["dH"][masked] == 0.0)
    np.testing.assert_allclose(b["dW"].sum(axis=0), 0.0, atol=1e-12)


def test_masked_rows_never_read():
    H, W, ids, a, mask = _rand_problem()
    masked = np.nonzero(mask == 0)[0]
    ids2, a2 = ids.copy(), a.copy()
    ids2[masked] = -1
    a2[masked] = np.nan
    f1, f2 = oracle.kd_forward(H, W, ids, a, mask), oracle.kd_forward(H, W, ids2, a2, mask)
    assert f1["loss"] == f2["loss"]
    b1, b2 = oracle.kd_backward(H, W, ids, a, mask), oracle.kd_backward(H, W, ids2, a2, mask)
    assert np.array_equal(b1["dH"], b2["dH"]) and np.array_equal(b1["dW"], b2["dW"])


def test_shift_invariances():
    H, W, ids, a, mask = _rand_problem()
    f = oracle.kd_forward(H, W, ids, a, mask)
    # teacher logits + c per row
    f2 = oracle.kd_forward(H, W, ids, a + np.arange(a.shape[0])[:, None] * 0.37, mask)
    assert abs(f2["loss"] - f["loss"]) <= 1e-12 * f["loss"]
    # every vocab row of W shifted by the same vector u: z_iv + h_i.u for all v
    u = np.random.default_rng(2).standard_normal(W.shape[1])
    f3 = oracle.kd_forward(H, W + u[None, :], ids, a, mask)
    assert abs(f3["loss"] - f["loss"]) <= 1e-11 * f["loss"]


def test_g_linearity():
    H, W, ids, a, mask = _rand_problem()
    b1 = oracle.kd_backward(H, W, ids, a, mask, g=1.0)
    b2 = oracle.kd_backward(H, W, ids, a, mask, g=0.37)
    np.testing.assert_allclose(b2["dH"], 0.37 * b1["dH"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(b2["dW"], 0.37 * b1["dW"], rtol=1e-13, atol=1e-16)


def test_k_permutation_permutes_gather():
    H, W, ids, a, mask = _rand_problem()
    perm = np.random.default_rng(3).permutation(ids.shape[1])
    f1 = oracle.kd_forward(H, W, ids, a, mask)
    f2 = oracle.kd_forward(H, W, ids[:, perm], a[:, perm], mask)
    assert np.array_equal(f2["zg"], f1["zg"][:, perm])
    assert abs(f2["loss"] - f1["loss"]) <= 1e-13 * f1["loss"]


def test_row_blocking_and_subsets_agree():
    H, W, ids, a, mask = _rand_problem()
    full = oracle.kd_forward(H, W, ids, a, mask, block=256)
    for blk in (1, 7, H.shape[0]):
        f = oracle.kd_forward(H, W, ids, a, mask, block=blk)
        np.testing.assert_allclose(f["lse"], full["lse"], rtol=1e-15)
        np.testing.assert_allclose(f["row_loss"], full["row_loss"], rtol=1e-15, atol=1e-300)
    rows = np.array([0, 5, 17, 39])
    sub = oracle.kd_forward(H, W, ids, a, mask, rows=rows)
    np.testing.assert_allclose(sub["lse"], full["lse"][rows], rtol=1e-15)
    bfull = oracle.kd_backward(H, W, ids, a, mask)
    bsub = oracle.kd_backward(H, W, ids, a, mask, rows=rows)
    np.testing.assert_allclose(bsub["dH"], bfull["dH"][rows], rtol=1e-13, atol=1e-16)


def test_duplicate_ids_add_term_by_term():
    """A repeated id contributes one term per occurrence (finite differences)."""
    H, W, ids, a, _ = tiny_problem(2, 3, 6, 3, 21)
    ids[0, 2] = ids[0, 0]
    b = oracle.kd_backward(H, W, ids, a)
    eps = 1e-6
    fd = np.zeros_like(W)
    for j in range(W.shape[0]):
        for c in range(W.shape[1]):
            Wp, Wm = W.copy(), W.copy()
            Wp[j, c] += eps
            Wm[j, c] -= eps
            fd[j, c] = (oracle.kd_forward(H, Wp, ids, a)["loss"] -
                        oracle.kd_forward(H, Wm, ids, a)["loss"]) / (2 * eps)
    assert rel(b["dW"], fd) <= 1e-7


# --------------------------------------------------------------------------
# library routines
# --------------------------------------------------------------------------
def test_scipy_logsumexp_and_rel_entr():
    H, W, ids, a, mask = _rand_problem()
    f = oracle.kd_forward(H, W, ids, a, mask)
    z = H @ W.T
    np.testing.assert_allclose(f["lse"], sps.logsumexp(z, axis=1), rtol=1e-14)
    live = np.nonzero(mask)[0]
    p = sps.softmax(a[live], axis=1)
    logq = z[live] - sps.logsumexp(z[live], axis=1, keepdims=True)
    q_t = np.exp(np.take_along_axis(logq, ids[live], axis=1))
    ref = sps.rel_entr(p, q_t).sum()
    assert abs(f["loss"] - ref) <= 1e-12 * ref


def test_torch_fp64_autograd():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    H, W, ids, a, mask = _rand_problem()
    g = 0.37
    Ht = torch.tensor(H, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    live = torch.tensor(np.nonzero(mask)[0])
    logq = F.log_softmax(Ht @ Wt.T, dim=1)
    logq_t = torch.gather(logq[live], 1, torch.tensor(ids)[live])
    p = torch.softmax(torch.tensor(a, dtype=torch.float64)[live], dim=1)
    L = F.kl_div(logq_t, p, reduction="sum")
    (g * L).backward()
    f = oracle.kd_forward(H, W, ids, a, mask)
    b = oracle.kd_backward(H, W, ids, a, mask, g=g)
    assert abs(f["loss"] - L.item()) <= 1e-12 * L.item()
    assert rel(b["dH"], Ht.grad.numpy()) <= 1e-12
    assert rel(b["dW"], Wt.grad.numpy()) <= 1e-12


# --------------------------------------------------------------------------
# temperature
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tau", [0.5, 1.7, 4.0])
def test_temperature_is_a_rescaling(tau):
    """L_tau(H, a) = tau^2 L_1(H / tau, a / tau), dH_tau = tau dH_1(H / tau),
    dW_tau = tau^2 dW_1(H / tau): the tempered loss against the plain one."""
    H, W, ids, a, mask = _rand_problem()
    g = 0.37
    f = oracle.kd_forward(H, W, ids, a, mask, tau=tau)
    b = oracle.kd_backward(H, W, ids, a, mask, g=g, tau=tau)
    f1 = oracle.kd_forward(H / tau, W, ids, a / tau, mask)
    b1 = oracle.kd_backward(H / tau, W, ids, a / tau, mask, g=g)
    assert abs(f["loss"] - tau * tau * f1["loss"]) <= 1e-12 * abs(f["loss"])
    np.testing.assert_allclose(f["lse"], f1["lse"], rtol=1e-13)
    np.testing.assert_allclose(f["zg"], tau * f1["zg"], rtol=1e-13, atol=1e-13)
    assert rel(b["dH"], tau * b1["dH"]) <= 1e-12
    assert rel(b["dW"], tau * tau * b1["dW"]) <= 1e-12


def test_temperature_torch_fp64_autograd():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    H, W, ids, a, mask = _rand_problem()
    g, tau = 0.37, 2.3
    Ht = torch.tensor(H, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    live = torch.tensor(np.nonzero(mask)[0])
    logq = F.log_softmax((Ht @ Wt.T) / tau, dim=1)
    logq_t = torch.gather(logq[live], 1, torch.tensor(ids)[live])
    p = torch.softmax(torch.tensor(a, dtype=torch.float64)[live] / tau, dim=1)
    L = tau * tau * F.kl_div(logq_t, p, reduction="sum")
    (g * L).backward()
    f = oracle.kd_forward(H, W, ids, a, mask, tau=tau)
    b = oracle.kd_backward(H, W, ids, a, mask, g=g, tau=tau)
    assert abs(f["loss"] - L.item()) <= 1e-12 * L.item()
    assert rel(b["dH"], Ht.grad.numpy()) <= 1e-12
    assert rel(b["dW"], Wt.grad.numpy()) <= 1e-12


def test_temperature_one_is_the_plain_loss():
    H, W, ids, a, mask = _rand_problem()
    f, f1 = oracle.kd_forward(H, W, ids, a, mask, tau=1.0), oracle.kd_forward(H, W, ids, a, mask)
    assert f["loss"] == f1["loss"] and np.array_equal(f["lse"], f1["lse"])


# --------------------------------------------------------------------------
# dW on a subset of vocabulary rows, from a given lse (full-size checks)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_dw_vocab_rows_matches_bruteforce_gradient(case):
    """Rows of dW formed from the brute-force lse agree with the 50-digit
    central-difference gradient, for every vocabulary row and for a subset."""
    H, W = np.array(case["H"]), np.array(case["W"])
    ids, a = np.array(case["t_ids"]), np.array(case["t_logits"])
    mask = None
    if case["masked"]:
        mask = np.ones(case["n"], np.uint8)
        mask[case["masked"]] = 0
    lse = [float(mpmath.mpf(x)) for x in case["lse"]]
    ref = _arr(case["dW"])
    tau = case.get("tau", 1.0)
    allv = np.arange(W.shape[0])
    got = oracle.dw_vocab_rows(H, W, "f64", ids, a, mask, lse, allv, g=case["g"], tau=tau)
    assert rel(got, ref) <= 1e-12
    sub = allv[::-2]
    got = oracle.dw_vocab_rows(H, W, "f64", ids, a, mask, lse, sub, g=case["g"], tau=tau, block=1)
    assert rel(got, ref[sub]) <= 1e-12


def test_dw_vocab_rows_bf16_storage_and_torch_autograd():
    """bf16-stored inputs (uint16 bit patterns) widened block by block: the
    selected rows equal torch fp64 autograd of the tempered loss."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    n, d, v, k, g, tau = 23, 8, 40, 6, 0.61, 1.9
    Hb = torch.randn(n, d).to(torch.bfloat16)
    Wb = (0.4 * torch.randn(v, d)).to(torch.bfloat16)
    ids = np.stack([rng.permutation(v)[:k] for _ in range(n)]).astype(np.int32)
    ids[4, 2] = ids[4, 0]                       # a repeated id adds term by term
    a = 2.0 * rng.standard_normal((n, k))
    mask = (rng.random(n) > 0.25).astype(np.uint8)
    Ht = Hb.double().requires_grad_(True)
    Wt = Wb.double().requires_grad_(True)
    live = torch.tensor(np.nonzero(mask)[0])
    logq = F.log_softmax((Ht @ Wt.T) / tau, dim=1)
    logq_t = torch.gather(logq[live], 1, torch.tensor(ids, dtype=torch.int64)[live])
    p = torch.softmax(torch.tensor(a)[live] / tau, dim=1)
    L = tau * tau * (p * (torch.log(p) - logq_t)).sum()
    (g * L).backward()
    lse = torch.logsumexp((Ht @ Wt.T) / tau, dim=1).detach().numpy()
    hs = Hb.view(torch.int16).numpy().view(np.uint16)
    ws = Wb.view(torch.int16).numpy().view(np.uint16)
    sub = np.array([ids[4, 0], 0, 39, 17, ids[0, 1]])
    sub = np.unique(sub)
    got = oracle.dw_vocab_rows(hs, ws, "bf16", ids, a, mask, lse, sub, g=g, tau=tau, block=5)
    assert rel(got, Wt.grad.numpy()[sub]) <= 1e-12
    with pytest.raises(ValueError):
        oracle.dw_vocab_rows(hs, ws, "bf16", ids, a, mask, lse, [3, 3], g=g, tau=tau)
