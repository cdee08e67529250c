"""Pins of the teacher-record check oracle (oracle/validate.py), CPU only.

The check counts unmasked rows holding an id outside [0, v) and rows holding
an id more than once, and reports the first row of each kind.  Pinned by
  * hand-built records with known answers (each fault alone, both in one row,
    faults on masked rows, K = 1, the edges -1 / 0 / v-1 / v);
  * a vectorised numpy restatement on random records (range by comparison,
    repeats by sorting each row and comparing neighbours);
  * planted mistakes in the oracle's source, each failing a pin.
"""
import types

import numpy as np
import pytest

import oracle.validate as ov
from oracle import validate_teacher


def test_valid_record():
    ids = np.array([[0, 1, 2], [9, 5, 7], [3, 8, 4]])
    assert validate_teacher(ids, 10) == (0, 0, -1, -1)


def test_each_fault_alone_and_together():
    v = 10
    ids = np.array([[0, 1, 2],     # ok
                    [0, 10, 2],    # id == v: out of range
                    [4, 4, 5],     # repeated
                    [-1, 3, -1],   # out of range and repeated
                    [9, 8, 0]])    # ok (edges 0 and v-1)
    assert validate_teacher(ids, v) == (2, 2, 1, 2)


def test_masked_rows_are_skipped():
    ids = np.array([[0, 0], [11, 1], [2, 3], [5, 5]])
    mask = np.array([0, 0, 1, 1], dtype=np.uint8)
    assert validate_teacher(ids, 10, mask) == (0, 1, -1, 3)
    assert validate_teacher(ids, 10, np.zeros(4, np.uint8)) == (0, 0, -1, -1)


def test_k1_never_repeats():
    ids = np.array([[3], [3], [-5], [0]])
    assert validate_teacher(ids, 4) == (1, 0, 2, -1)


def test_empty():
    assert validate_teacher(np.zeros((0, 5), np.int64), 10) == (0, 0, -1, -1)


def _vectorised(ids, v, mask):
    live = np.ones(ids.shape[0], bool) if mask is None else mask != 0
    rng_bad = ((ids < 0) | (ids >= v)).any(axis=1) & live
    s = np.sort(ids, axis=1)
    rep_bad = (s[:, 1:] == s[:, :-1]).any(axis=1) & live
    first = lambda b: int(np.flatnonzero(b)[0]) if b.any() else -1  # noqa: E731
    return int(rng_bad.sum()), int(rep_bad.sum()), first(rng_bad), first(rep_bad)


@pytest.mark.parametrize("seed", range(4))
def test_against_vectorised_restatement(seed):
    rng = np.random.default_rng(seed)
    n, k, v = 300, 12, 200
    ids = rng.integers(-3, v + 3, size=(n, k))
    mask = (rng.random(n) < 0.8).astype(np.uint8) if seed % 2 else None
    assert validate_teacher(ids, v, mask) == _vectorised(ids, v, mask)


SRC = open(ov.__file__).read()
MUTATIONS = [
    ("upper edge", "x >= v", "x > v"),
    ("lower edge", "x < 0 or", "x < -1 or"),
    ("mask ignored", "if mask is not None and int(mask[i]) == 0:", "if False:"),
    ("last row first", "if first_range < 0:", "if True:"),
    ("repeat test", "len(set(row)) < len(row)", "len(set(row)) < len(row) - 1"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutations_are_caught(name, old, new):
    assert old in SRC
    mod = types.ModuleType("validate_mutant")
    exec(compile(SRC.replace(old, new), ov.__file__ + "<mutant>", "exec"), mod.__dict__)
    cases = [(np.array([[0, 1, 2], [0, 10, 2], [4, 4, 5], [-1, 3, -1], [9, 8, 0], [10, 1, 1]]), 10, None),
             (np.array([[0, 0], [11, 1], [2, 3], [5, 5]]), 10, np.array([0, 0, 1, 1], np.uint8))]
    caught = any(mod.validate_teacher(ids, v, m) != validate_teacher(ids, v, m) for ids, v, m in cases)
    assert caught, f"mutation '{name}' not caught"
