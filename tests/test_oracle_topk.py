"""Pins of the teacher top-K oracle (oracle/topk.py), CPU only.

The oracle keeps, per position, the K largest teacher logits with their ids,
largest first, equal logits ordered by the lower id.  It is pinned against
things other than itself:
  * brute force: logits as explicit Python sums and the record as Python's
    ``sorted`` on (-z, id) over all V, on tiny inputs;
  * hand-computed answers: an identity projection (z = h), equal logits
    (the K lowest ids), a two-valued row;
  * invariants on random inputs: descending logits, distinct ids, every id
    left out at most the K-th logit, the set equal to numpy's argpartition
    set when no ties are possible;
  * planted mistakes in the oracle's source must fail at least one pin.
"""
import types

import numpy as np
import pytest

import oracle.topk as tk
from oracle import teacher_topk


def _brute(H, W, k):
    ids, vals = [], []
    for h in H:
        z = [sum(float(a) * float(b) for a, b in zip(h, w)) for w in W]
        order = sorted(range(len(W)), key=lambda v: (-z[v], v))[:k]
        ids.append(order)
        vals.append([z[v] for v in order])
    return np.array(ids), np.array(vals)


@pytest.mark.parametrize("seed,n,d,v,k", [(0, 5, 3, 11, 4), (1, 3, 6, 20, 20), (2, 4, 2, 9, 1), (3, 6, 4, 30, 7)])
def test_against_brute_force(seed, n, d, v, k):
    rng = np.random.default_rng(seed)
    H = rng.integers(-3, 4, size=(n, d)).astype(np.float64)  # integer values: ties occur
    W = rng.integers(-3, 4, size=(v, d)).astype(np.float64)
    ids, vals = teacher_topk(H, W, k)
    bids, bvals = _brute(H, W, k)
    np.testing.assert_array_equal(ids, bids)
    np.testing.assert_array_equal(vals, bvals)


def test_identity_projection():
    h = np.array([[0.5, -1.0, 2.0, 2.0, 0.0, 3.5]])
    ids, vals = teacher_topk(h, np.eye(6), 4)
    np.testing.assert_array_equal(ids, [[5, 2, 3, 0]])  # 2.0 twice: id 2 before id 3
    np.testing.assert_array_equal(vals, [[3.5, 2.0, 2.0, 0.5]])


def test_equal_logits_keep_lowest_ids():
    H = np.ones((2, 4))
    W = np.zeros((50, 4))
    ids, vals = teacher_topk(H, W, 7)
    np.testing.assert_array_equal(ids, np.tile(np.arange(7), (2, 1)))
    assert np.all(vals == 0.0)


def test_two_valued_row():
    # columns 10..19 hold 1, the rest 0: the record is ids 10..19 then 0, 1, ...
    W = np.zeros((40, 1))
    W[10:20, 0] = 1.0
    ids, vals = teacher_topk(np.ones((1, 1)), W, 13)
    np.testing.assert_array_equal(ids[0], list(range(10, 20)) + [0, 1, 2])
    np.testing.assert_array_equal(vals[0], [1.0] * 10 + [0.0] * 3)


def test_invariants_random():
    rng = np.random.default_rng(7)
    H = rng.standard_normal((20, 16))
    W = rng.standard_normal((500, 16))
    k = 30
    ids, vals = teacher_topk(H, W, k, block=7)
    Z = H @ W.T  # another BLAS blocking than the oracle's: equal up to the last bits
    for i in range(20):
        assert np.all(np.diff(vals[i]) <= 0)
        assert len(set(ids[i].tolist())) == k
        np.testing.assert_allclose(vals[i], Z[i, ids[i]], rtol=1e-12, atol=1e-12)
        rest = np.setdiff1d(np.arange(500), ids[i])
        assert Z[i, rest].max() <= vals[i, -1] + 1e-12
        assert set(np.argpartition(-Z[i], k)[:k].tolist()) == set(ids[i].tolist())


SRC = open(tk.__file__).read()
MUTATIONS = [
    ("ascending", "order = np.lexsort((cols, -z))[:k]", "order = np.lexsort((cols, z))[:k]"),
    ("tie to higher id", "order = np.lexsort((cols, -z))[:k]", "order = np.lexsort((-cols, -z))[:k]"),
    ("one short", "order = np.lexsort((cols, -z))[:k]", "order = np.lexsort((cols, -z))[1:k + 1]"),
    ("transposed operand", "Z = H[r0:r0 + block] @ W.T", "Z = H[r0:r0 + block] @ W[::-1].T"),
    ("ties ignored", "order = np.lexsort((cols, -z))[:k]", "order = np.argsort(-z, kind='quicksort')[:k]"),
]


def _mutant(old, new):
    assert old in SRC
    mod = types.ModuleType("topk_mutant")
    exec(compile(SRC.replace(old, new), tk.__file__ + "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutations_are_caught(name, old, new):
    mod = _mutant(old, new)
    caught = False
    rng = np.random.default_rng(11)
    cases = [(rng.integers(-3, 4, size=(4, 3)).astype(float), rng.integers(-3, 4, size=(25, 3)).astype(float), 6)]
    cases.append((np.ones((1, 4)), np.zeros((50, 4)), 7))
    for H, W, k in cases:
        try:
            ids, vals = mod.teacher_topk(H, W, k)
        except Exception:
            caught = True
            break
        bids, bvals = _brute(H, W, k)
        if not (np.array_equal(ids, bids) and np.array_equal(vals, bvals)):
            caught = True
            break
    assert caught, f"mutation '{name}' not caught"
