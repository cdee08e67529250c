"""Peak device memory of the fused chunked loss is linear in the number of
positions N, with the slope of the caller's per-position buffers only.

The method keeps one chunk of the positions x vocabulary grid at a time, so
its memory grows only through the per-position inputs and outputs (the pages'
long-context comparison of the fully chunked loss against the next-best
chunked variant: agentlenshq.com, "LLMのための効率的な知識蒸留…", section
"ロングコンテキストへのスケーリング"; aivibenews.ru, section "Что на одной
карте").  The workspace is a function of (chunk, D, V, K, dtypes), never of N.

At the long-context shapes (D = 4096, V = 128256, K = 100, chunk 4096, bf16)
the per-position bytes are H (2D) + dH (4D) + teacher ids (4K) + teacher
logits (2K) + lse (4) = 25180 B; the intercept is W (2VD) + dW (4VD) + the
workspace.  Peak is taken with torch's allocator statistics after inputs are
resident (outputs, workspace and everything the two calls touch included).
"""
import numpy as np
import pytest
import torch

from chunked_kl_loss_row_amd import binding as B
from chunked_kl_loss_row_amd import loss as L

pytestmark = pytest.mark.gpu

D, V, K, C = 4096, 128256, 100, 4096
PER_ROW = 2 * D + 4 * D + 4 * K + 2 * K + 4


def _peak_bytes(n, W, dW):
    g = torch.Generator(device="cuda")
    g.manual_seed(n)
    H = torch.randn(n, D, device="cuda", dtype=torch.bfloat16, generator=g)
    rows = torch.arange(n, device="cuda", dtype=torch.int64)[:, None]
    ks = torch.arange(K, device="cuda", dtype=torch.int64)[None, :]
    ids = ((rows * 7919 + ks * 1283) % V).to(torch.int32)  # distinct in a row: 1283 * (K - 1) < V
    lg = (3.0 * torch.randn(n, K, device="cuda", generator=g)).to(torch.bfloat16)
    del rows, ks
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    prob = L.make_problem(H, W, ids, lg, C)
    ws = L.workspace_for(prob, H.device)
    loss = torch.empty(1, device="cuda")
    lse = torch.empty(n, device="cuda")
    dH = torch.empty(n, D, device="cuda")
    B.kd_chunked_fwd(prob, H, W, ids, lg, None, loss, lse, None, None, ws)
    B.kd_chunked_bwd(prob, H, W, ids, lg, None, lse, None, dH, dW, ws)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    inputs = base - (W.numel() * 2 + dW.numel() * 4)  # per-row inputs resident before the reset
    ws_bytes = ws.numel()
    ok = bool(torch.isfinite(loss).item())
    del H, ids, lg, ws, loss, lse, dH
    torch.cuda.empty_cache()
    return peak, inputs, ws_bytes, ok


def test_peak_memory_linear_in_n():
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    W = (0.02 * torch.randn(V, D, device="cuda", generator=g)).to(torch.bfloat16)
    dW = torch.zeros(V, D, device="cuda")
    ns = [16384, 32768, 65536, 131072, 262144]
    peaks, wss = [], []
    for n in ns:
        peak, inputs, ws_bytes, ok = _peak_bytes(n, W, dW)
        assert ok
        peaks.append(peak)
        wss.append(ws_bytes)
        print(f"n={n}: peak {peak / 2**30:.3f} GiB (per-row inputs {inputs / 2**30:.3f} GiB, "
              f"workspace {ws_bytes / 2**30:.3f} GiB); dense fp32 z + dZ would be "
              f"{2 * n * V * 4 / 2**30:.1f} GiB", flush=True)
    assert len(set(wss)) == 1, "workspace must not depend on n"
    slope, icpt = np.polyfit(np.array(ns, dtype=np.float64), np.array(peaks, dtype=np.float64), 1)
    resid = np.array(peaks, dtype=np.float64) - (icpt + slope * np.array(ns, dtype=np.float64))
    print(f"fit: {icpt / 2**30:.4f} GiB + {slope:.2f} B x n (predicted slope {PER_ROW} B); "
          f"max |residual| {np.abs(resid).max() / 2**20:.3f} MiB", flush=True)
    # allocations are rounded to 512 B per tensor: the fit is exact up to that
    assert abs(slope - PER_ROW) <= 0.001 * PER_ROW
    assert np.abs(resid).max() <= 2**20
    expect_icpt = V * D * 2 + V * D * 4 + wss[0]
    assert abs(icpt - expect_icpt) <= 8 * 2**20
