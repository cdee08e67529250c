"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutation edits one line of ``oracle/kd_oracle.py``'s source text (a
dropped term, a wrong sign, a wrong index, a transposed operand, an inverted
mask), loads the edited copy as a separate module, and runs the pins that do
not depend on the oracle itself: the 50-digit brute-force fixture (values and
central-difference gradients, at temperature 1 and at three other
temperatures, also for the dW rows formed from a given lse), the zero-loss
construction and the dZ sum-to-zero invariant.  Every mutation must fail at least one of them.
"""
import json
import os
import types

import mpmath
import numpy as np
import pytest

import oracle.kd_oracle as kd

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = open(kd.__file__).read()

MUTATIONS = [
    ("teacher not renormalised", "p = e / e.sum(axis=1, keepdims=True)", "p = e"),
    ("entropy sign", "np.where(p > 0.0, p * np.log(p), 0.0)", "np.where(p > 0.0, -p * np.log(p), 0.0)"),
    ("lse drops the max", "return m + np.log(np.exp(z - m[:, None]).sum(axis=1))",
     "return np.log(np.exp(z - m[:, None]).sum(axis=1))"),
    ("lse is the max", "return m + np.log(np.exp(z - m[:, None]).sum(axis=1))", "return m"),
    ("wrong vocab row", "return h_rows @ w.T", "return h_rows @ np.roll(w, 1, axis=0).T"),
    ("gather sign", "(negent - (p * zg_b).sum(axis=1) / tau + s * lse_b[li])",
     "(negent + (p * zg_b).sum(axis=1) / tau + s * lse_b[li])"),
    ("dropped entropy term", "(negent - (p * zg_b).sum(axis=1) / tau + s * lse_b[li])",
     "(- (p * zg_b).sum(axis=1) / tau + s * lse_b[li])"),
    ("dropped lse term", "(negent - (p * zg_b).sum(axis=1) / tau + s * lse_b[li])",
     "(negent - (p * zg_b).sum(axis=1) / tau)"),
    ("gather off by one", "np.take_along_axis(z[li], np.where(inside, ids, 0), axis=1)",
     "np.take_along_axis(z[li], np.where(inside, (ids + 1) % z.shape[1], 0), axis=1)"),
    ("unmatched ids wrap in the gather", "inside = (ids >= 0) & (ids < z.shape[1])",
     "inside = np.ones(ids.shape, dtype=bool); ids = ids % z.shape[1]"),
    ("unmatched ids wrap in the scatter", "inside = (ids_b >= 0) & (ids_b < V)",
     "inside = np.ones(ids_b.shape, dtype=bool); ids_b = ids_b % V"),
    ("mask inverted", "return (np.asarray(mask)[rows] != 0).astype(np.float64)",
     "return (np.asarray(mask)[rows] == 0).astype(np.float64)"),
    ("scatter sign", "-p.ravel()[inside])", "p.ravel()[inside])"),
    ("scatter dropped", "np.add.at(dz, (r_idx", "(lambda *a: None)(dz, (r_idx"),
    ("softmax not normalised", "dz = s[:, None] * np.exp(z - lse_b[:, None])",
     "dz = s[:, None] * np.exp(z)"),
    ("g ignored", "dz *= g", "dz *= 1.0"),
    ("dH transposed operand", "dH[b0 + live] = dz @ W", "dH[b0 + live] = dz @ W[::-1]"),
    ("dW wrong rows", "dW += dz.T @ hs", "dW += dz.T @ hs[::-1]"),
    # temperature handling (caught by the tau != 1 brute-force cases)
    ("tau^2 dropped", "row_loss[b0 + li] = tau * tau * (", "row_loss[b0 + li] = ("),
    ("teacher not tempered", "a = np.asarray(t_logits, dtype=np.float64) / tau",
     "a = np.asarray(t_logits, dtype=np.float64)"),
    ("student lse not tempered", "lse_b = row_logsumexp(z / tau)", "lse_b = row_logsumexp(z)"),
    ("gathered logit not tempered", "(p * zg_b).sum(axis=1) / tau", "(p * zg_b).sum(axis=1)"),
    ("backward logits not tempered", "z = student_logits(hs, W) / tau", "z = student_logits(hs, W)"),
    ("gradient tau factor dropped", "dz *= g * tau", "dz *= g"),
    # dW on a subset of vocabulary rows from a given lse
    ("vocab rows: scatter sign", "np.add.at(dz, (r, j[r, kk]), -p[r, kk])",
     "np.add.at(dz, (r, j[r, kk]), p[r, kk])"),
    ("vocab rows: lse ignored", "dz = s[:, None] * np.exp(z - lse[live][:, None])",
     "dz = s[:, None] * np.exp(z)"),
    ("vocab rows: shifted W rows", "Wv = widen(W_stored[vocab], x_dtype)",
     "Wv = widen(W_stored[(vocab + 1) % V], x_dtype)"),
    ("vocab rows: tau factor dropped", "out += (g * tau) * (dz.T @ hs)", "out += g * (dz.T @ hs)"),
    ("vocab rows: mask ignored", "live_all = np.nonzero(_mask_rows(mask, np.arange(n)) != 0)[0]",
     "live_all = np.arange(n)"),
    ("vocab rows: column map reversed", "col[vocab] = np.arange(vocab.size)",
     "col[vocab] = np.arange(vocab.size)[::-1]"),
    ("vocab rows: student not tempered", "z = student_logits(hs, Wv) / tau", "z = student_logits(hs, Wv)"),
]


def _load_mutant(old, new):
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("kd_mutant")
    mod.__file__ = kd.__file__
    exec(compile(SRC.replace(old, new), kd.__file__ + "<mutant>", "exec"), mod.__dict__)
    return mod


def _golden():
    cases = []
    for name in ("tiny_bruteforce.json", "tiny_bruteforce_tau.json"):
        with open(os.path.join(HERE, "golden", name)) as f:
            cases += json.load(f)["cases"]
    return cases


def _f(x):
    with mpmath.workdps(50):
        return float(mpmath.mpf(x))


def pins(mod):
    """Run the independent pins against module ``mod``; raise on any failure."""
    for c in _golden():
        H, W = np.array(c["H"]), np.array(c["W"])
        ids, a = np.array(c["t_ids"]), np.array(c["t_logits"])
        mask = None
        if c["masked"]:
            mask = np.ones(c["n"], np.uint8)
            mask[c["masked"]] = 0
        tau = c.get("tau", 1.0)
        f = mod.kd_forward(H, W, ids, a, mask, tau=tau)
        L = _f(c["loss"])
        assert abs(f["loss"] - L) <= 1e-12 * abs(L)
        np.testing.assert_allclose(f["lse"], [_f(x) for x in c["lse"]], rtol=1e-13)
        b = mod.kd_backward(H, W, ids, a, mask, g=c["g"], want_dz=True, tau=tau)
        dH = np.array([[_f(x) for x in r] for r in c["dH"]])
        dW = np.array([[_f(x) for x in r] for r in c["dW"]])
        assert np.linalg.norm(b["dH"] - dH) <= 1e-10 * np.linalg.norm(dH)
        assert np.linalg.norm(b["dW"] - dW) <= 1e-10 * np.linalg.norm(dW)
        # each dZ row sums to zero when every id of the row matches a column
        # (an unmatched id leaves its p out of the scatter: the row sums to it)
        matched = np.all((ids >= 0) & (ids < W.shape[0]), axis=1)
        np.testing.assert_allclose(b["dZ"].sum(axis=1)[matched], 0.0, atol=1e-13)
        if not matched.all():
            p = np.exp(a - a.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            live = np.ones(c["n"], bool) if mask is None else mask != 0
            left = c["g"] * np.where((ids >= 0) & (ids < W.shape[0]), 0.0, p).sum(axis=1) * live
            np.testing.assert_allclose(b["dZ"].sum(axis=1), left, atol=1e-13)
        sub = np.arange(W.shape[0])[::-2]
        dWs = mod.dw_vocab_rows(H, W, "f64", ids, a, mask, [_f(x) for x in c["lse"]], sub,
                                g=c["g"], tau=tau, block=2)
        assert np.linalg.norm(dWs - dW[sub]) <= 1e-10 * np.linalg.norm(dW[sub])
    # zero-loss construction
    v = d = 64
    rng = np.random.default_rng(7)
    ids = np.stack([rng.permutation(v)[:5] for _ in range(4)])
    a = -np.sort(-3.0 * rng.standard_normal((4, 5)), axis=1)
    H = np.full((4, d), -1e4)
    for i in range(4):
        H[i, ids[i]] = a[i]
    assert abs(mod.kd_forward(H, np.eye(v), ids, a)["loss"]) <= 1e-12


def test_unmutated_oracle_passes_pins():
    pins(_load_mutant("", ""))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        pins(mod)
