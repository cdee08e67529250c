"""GPU tests of the teacher-record check (kd_chunked_validate) against the
oracle (oracle/validate.py).  Counts and first rows are integers: they must
agree exactly."""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_row_amd import inputs
from chunked_kl_loss_row_amd import loss as L
from gpu_helpers import log

pytestmark = pytest.mark.gpu

I32_MIN, I32_MAX = -2 ** 31, 2 ** 31 - 1


def _run(ids, v, mask=None):
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()
    out = L.validate_teacher(t, v, m)
    torch.cuda.synchronize()
    return tuple(int(x) for x in out.cpu().tolist())


def _plant(ids, v, seed, count):
    """Copy of ids with faults in seeded rows: out-of-range values at the
    edges, and repeats at the first/last/adjacent positions."""
    rng = np.random.default_rng(seed)
    ids = ids.copy()
    n, k = ids.shape
    rows = rng.choice(n, size=count, replace=False)
    for r in rows:
        kind = rng.integers(0, 6)
        if kind == 0:
            ids[r, rng.integers(0, k)] = v
        elif kind == 1:
            ids[r, rng.integers(0, k)] = -1
        elif kind == 2:
            ids[r, rng.integers(0, k)] = rng.choice([I32_MIN, I32_MAX])
        elif k > 1 and kind == 3:
            ids[r, k - 1] = ids[r, 0]
        elif k > 1 and kind == 4:
            j = rng.integers(0, k - 1)
            ids[r, j + 1] = ids[r, j]
        else:
            ids[r, 0] = -7
            if k > 1:
                ids[r, 1] = -7
    return ids


@pytest.mark.parametrize("name", ["gpt-oss-20b-32k", "gpt-oss-120b-b4x32k", "tiny-f32"])
def test_valid_records_pass(name):
    wl = inputs.workload(name)
    n = min(wl.n, 8192)
    inp = inputs.make_inputs(wl, seed=1, n=n, only=("t_ids", "mask"))
    log(f"case valid record {name} n={n}")
    assert _run(inp["t_ids"], wl.v, inp.get("mask")) == (0, 0, -1, -1)


@pytest.mark.parametrize("k,masked", [(100, False), (100, True), (256, False), (1, True), (3, False)])
def test_planted_faults_match_oracle(k, masked):
    n, v = 5000, 201088
    wl = inputs.custom(n, 64, v, k, 512, tag=700 + k)
    ids = inputs.make_inputs(wl, seed=3, only=("t_ids",))["t_ids"]
    bad = _plant(ids, v, seed=k, count=60)
    mask = (np.random.default_rng(9).random(n) < 0.7).astype(np.uint8) if masked else None
    log(f"case planted faults k={k} masked={masked}")
    got = _run(bad, v, mask)
    want = oracle.validate_teacher(bad, v, mask)
    assert got == want and got[0] + got[1] > 0


def test_empty_and_all_masked():
    assert _run(np.zeros((0, 10), np.int32), 100) == (0, 0, -1, -1)
    ids = np.full((64, 4), -1, np.int32)
    assert _run(ids, 100, np.zeros(64, np.uint8)) == (0, 0, -1, -1)
    assert _run(ids, 100) == (64, 64, 0, 0)


def test_bool_mask_and_last_row():
    n, k, v = 1031, 7, 50
    ids = np.tile(np.arange(k, dtype=np.int32), (n, 1))
    ids[n - 1, 3] = 50
    t = torch.from_numpy(ids).cuda()
    m = torch.ones(n, dtype=torch.bool, device="cuda")
    out = L.validate_teacher(t, v, m)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [1, 0, n - 1, -1]
    m[n - 1] = False
    out = L.validate_teacher(t, v, m)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [0, 0, -1, -1]


def test_long_context_record():
    """The 262144-row teacher record of the long-context workload (65536
    workgroups): valid as generated; three planted faults found exactly."""
    wl = inputs.workload("long-256k")
    ids = inputs.make_inputs(wl, seed=0, only=("t_ids",))["t_ids"]
    log(f"case validate long-256k n={ids.shape[0]} k={ids.shape[1]}")
    assert _run(ids, wl.v) == (0, 0, -1, -1)
    bad = ids.copy()
    bad[7, 5] = wl.v
    bad[200000, 99] = bad[200000, 0]
    bad[262143, 50] = -1
    assert _run(bad, wl.v) == (2, 1, 7, 200000)
