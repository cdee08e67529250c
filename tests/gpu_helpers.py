"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI binding, and compare with the oracle."""
import sys

import numpy as np
import torch

from chunked_kl_loss_row_amd import loss as L


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(arr, tag=None):
    """Host array -> contiguous device tensor (uint16 bits -> bfloat16)."""
    if arr is None:
        return None
    if tag == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def upload(inp):
    wl = inp["wl"]
    return {
        "H": dev(inp["H"], wl.x_dtype),
        "W": dev(inp["W"], wl.x_dtype),
        "t_ids": dev(inp["t_ids"]),
        "t_logits": dev(inp["t_logits"], wl.t_dtype),
        "mask": dev(inp["mask"]) if inp["mask"] is not None else None,
    }


def run_hip(d, chunk, g=None, mask="default", dW_init=None, zg=True, row_loss=True, workspace=None,
            temperature=1.0):
    """Forward + backward on the GPU; returns numpy results."""
    m = d["mask"] if isinstance(mask, str) else mask
    f = L.forward(d["H"], d["W"], d["t_ids"], d["t_logits"], m, chunk=chunk, row_loss=row_loss, zg=zg,
                  workspace=workspace, temperature=temperature)
    gl = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda")
    dW = None if dW_init is None else dW_init.clone()
    dH, dW = L.backward(d["H"], d["W"], d["t_ids"], d["t_logits"], m, f["lse"], gl, dW=dW, chunk=chunk,
                        workspace=f["workspace"], temperature=temperature)
    torch.cuda.synchronize()
    out = {"loss": float(f["loss"].item()), "lse": f["lse"].cpu().numpy(), "dH": dH, "dW": dW}
    if row_loss:
        out["row_loss"] = f["row_loss"].cpu().numpy()
    if zg:
        out["zg"] = f["zg"].cpu().numpy()
    return out


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def vocab_sample(t_ids, mask, v, count, seed=0):
    """``count`` distinct seeded vocabulary ids: half from the teacher ids of
    unmasked rows, the rest uniform over the vocabulary (disjoint from the
    first half)."""
    rng = np.random.default_rng([seed, 71])
    live = t_ids if mask is None else t_ids[mask != 0]
    hit = np.unique(live)
    a = rng.choice(hit, size=min(count // 2, hit.size), replace=False)
    rest = np.setdiff1d(np.arange(v), a)
    b = rng.choice(rest, size=count - a.size, replace=False)
    return np.sort(np.concatenate([a, b])).astype(np.int64), a


def oracle_forward_all(inp, tau=1.0, slice_rows=4096, block=256, tag=""):
    """The oracle's forward (lse, row loss, gathered logits, loss) for every
    row of a stored input dict, in slices of rows with a progress line each
    (rows are independent, so the slices change nothing)."""
    import math

    import oracle

    wl = inp["wl"]
    n = inp["H"].shape[0]
    Wx = oracle.widen(inp["W"], wl.x_dtype)
    lse = np.empty(n)
    rl = np.empty(n)
    zg = np.empty((n, inp["t_ids"].shape[1]))
    for r0 in range(0, n, slice_rows):
        r1 = min(n, r0 + slice_rows)
        m = None if inp["mask"] is None else inp["mask"][r0:r1]
        f = oracle.kd_forward(oracle.widen(inp["H"][r0:r1], wl.x_dtype), Wx, inp["t_ids"][r0:r1],
                              oracle.widen(inp["t_logits"][r0:r1], wl.t_dtype), m, block=block, tau=tau)
        lse[r0:r1], rl[r0:r1], zg[r0:r1] = f["lse"], f["row_loss"], f["zg"]
        log(f"[{tag}] oracle forward rows {r1}/{n}")
    return {"lse": lse, "row_loss": rl, "zg": zg, "loss": math.fsum(rl.tolist())}
