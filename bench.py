#!/usr/bin/env python3
"""Benchmark of the fused chunked top-K KL loss (forward + backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over the workload: kd_chunked_fwd
(per pass of up to 8 chunks: teacher renormalisation, fused projection +
online logsumexp + top-K gather, merge, running-loss fold) then
kd_chunked_bwd (per group of --dw-chunks chunks, default 2: recomputed
projection + closed-form dZ, dH = dZ W, dW += dZ^T H).  Inputs are
seeded synthetic tensors already resident in HBM when timing starts; dW keeps
accumulating across steps (it is zeroed once, outside the timed region).

Prints ONE JSON line: tokens/s (value), TFLOP/s counted as 8*N*D*V per step
and its fraction of the bf16 dense matrix-core peak, peak HBM GiB, a roofline
record of the dominant kernel (per-kernel durations from HIP events recorded
on the launch stream during a second pass of the same steps; the headline
steps run without them), and the fp64 CPU oracle timed on a bounded sample of
the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
# vocabulary entries per projection tile of the library (its per-tile partials
# and tile bounds scale with ceil(V / this)); a CPU test checks it against the
# kernel sources
PROJ_TILE_V = 384
PEAK_BF16_TFLOPS = 2516.6   # dense bf16 matrix cores: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_F32_TFLOPS = 157.3     # dense fp32 matrix cores
PEAK_HBM_GBS = 8000.0

METRIC = "fused KL fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak); peak GiB"
GEMM_KINDS = ("fwd_proj", "bwd_dz", "bwd_dh", "bwd_dw")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt-oss-20b-32k")
    ap.add_argument("--chunk", type=int, default=None, help="override the workload's chunk size")
    ap.add_argument("--dw-chunks", type=int, default=2,
                    help="chunks the backward takes at once (kd_problem.dw_chunks): 2 keeps two chunks of dZ "
                         "in the workspace and reads/writes dW once per two chunks")
    ap.add_argument("--cpu-rows", type=int, default=3072, help="rows of the CPU oracle sample (about 15-20 s on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=None,
                    help="rocprofv3 FETCH_SIZE/WRITE_SIZE summary with a line per matrix-core kernel "
                         "(default: profiles/kd_gemms_<workload>_traffic.txt)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the single-call variant (kd_chunked_fwd_bwd)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor GEMM library (hipBLASLt through torch.mm) on the three GEMM "
                         "shapes of one backward group, bf16 in and out, for comparison")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy (y = -x, fp32) of this many MiB before warm-up: "
                         "the known-size dispatch that scales the memory counters of a --pmc run")
    return ap.parse_args()


def source_digest():
    """sha256 over the kernel sources: a traffic summary is valid only for the code it was taken on."""
    import hashlib

    h = hashlib.sha256()
    src = os.path.join(ROOT, "chunked_kl_loss_row_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(src, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(path, kernel):
    """HBM bytes per launch of ``kernel`` from a committed counter summary (lines
    ``traffic: <kernel> <scaled bytes per launch>`` under ``source_digest: <digest>``),
    or None when the summary is missing, has no line for the kernel or was taken on
    other kernel sources."""
    if not path or not os.path.exists(path):
        return None
    digest, found = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, _, v = line.partition(":")
            k, v = k.strip(), v.split()
            if k == "source_digest" and v:
                digest = v[0]
            elif k == "traffic" and len(v) >= 2 and v[0] == kernel:
                try:
                    found = int(float(v[1]))
                except ValueError:
                    return None
    return found if digest == source_digest() else None


def parse_sclk(text):
    """Current shader clock in MHz from the text of pp_dpm_sclk (the line marked
    with '*'), or None."""
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            part = line.split(":", 1)[-1].strip().rstrip("*").strip().lower()
            if part.endswith("mhz"):
                try:
                    return float(part[:-3])
                except ValueError:
                    return None
    return None


class ClockSampler:
    """Samples the GPU's current shader clock (pp_dpm_sclk in sysfs), and,
    where the card's hwmon entries exist, its board power (power1_input,
    microwatts, against power1_cap) and junction temperature (the temp*_input
    labelled "junction", millidegrees), from a background thread while the
    timed steps run.  At this load the chip runs at its power cap, so the
    clock it sustains differs from box to box; the sampled means are reported
    next to the step time as context."""

    def __init__(self, period_s=0.025):
        self.path = self._find()
        self.hwmon = self._find_hwmon(self.path)
        self.period_s = period_s
        self.samples = []
        self.power = []
        self.temp = []
        self._stop = None
        self._thread = None

    @staticmethod
    def _find():
        import glob
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        return cards[0] if len(cards) == 1 else None  # several GPUs: which one is ours is not checked

    @staticmethod
    def _find_hwmon(sclk_path):
        """(power1_input, power1_cap, junction temp*_input) of the card, or None
        (also on any error: the sensors are context, never a reason to fail)."""
        try:
            return ClockSampler._find_hwmon_paths(sclk_path)
        except Exception:
            return None

    @staticmethod
    def _find_hwmon_paths(sclk_path):
        import glob
        if not sclk_path:
            return None
        dev = os.path.dirname(sclk_path)
        for h in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
            pw, cap = os.path.join(h, "power1_input"), os.path.join(h, "power1_cap")
            temp = None
            for lab in sorted(glob.glob(os.path.join(h, "temp*_label"))):
                try:
                    if open(lab).read().strip() == "junction":
                        temp = lab[:-len("label")] + "input"
                except OSError:
                    pass
            if os.path.exists(pw):
                return pw, (cap if os.path.exists(cap) else None), temp
        return None

    @staticmethod
    def _read_int(path):
        try:
            with open(path) as f:
                return int(f.read().strip())
        except (OSError, ValueError, UnicodeDecodeError):
            return None

    def _run(self):
        # one sample before the first look at the stop flag, so every run has one
        while True:
            try:
                with open(self.path) as f:
                    mhz = parse_sclk(f.read())
                if mhz:
                    self.samples.append(mhz)
            except OSError:
                return
            if self.hwmon:
                w = self._read_int(self.hwmon[0])
                if w is not None:
                    self.power.append(w / 1e6)
                if self.hwmon[2]:
                    t = self._read_int(self.hwmon[2])
                    if t is not None:
                        self.temp.append(t / 1e3)
            if self._stop.wait(self.period_s):
                return

    def __enter__(self):
        import threading
        if self.path:
            self._stop = threading.Event()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        return {"mean": round(sum(self.samples) / len(self.samples), 1), "min": min(self.samples),
                "max": max(self.samples), "samples": len(self.samples), "source": self.path}

    def power_summary(self):
        """Board power (W) over the samples, with the card's power cap, or None."""
        if not self.power:
            return None
        cap = self._read_int(self.hwmon[1]) if self.hwmon and self.hwmon[1] else None
        return {"mean": round(sum(self.power) / len(self.power), 1), "min": round(min(self.power), 1),
                "max": round(max(self.power), 1), "cap": round(cap / 1e6, 1) if cap else None,
                "samples": len(self.power), "source": self.hwmon[0]}

    def temp_summary(self):
        """Junction temperature (degrees C) over the samples, or None."""
        if not self.temp:
            return None
        return {"mean": round(sum(self.temp) / len(self.temp), 1), "max": round(max(self.temp), 1),
                "samples": len(self.temp)}


def read_clock(path, kernel):
    """Shader clock (GHz) of ``kernel`` from a committed SQ-counter summary
    (rows ``kernel dur_ms cycles clk_GHz ...``), or None when the summary is
    missing or was taken on other kernel sources."""
    try:
        text = open(path).read()
    except OSError:
        return None
    dig = None
    for line in text.splitlines():
        if line.startswith("source_digest:"):
            dig = line.split(":", 1)[1].strip()
        parts = line.split()
        if len(parts) >= 4 and parts[0] == kernel and dig == source_digest():
            try:
                return float(parts[3])
            except ValueError:
                return None
    return None


def cpu_baseline(inp, rows_n):
    import numpy as np

    import oracle
    from chunked_kl_loss_row_amd import inputs

    wl = inp["wl"]
    rows = inputs.sample_rows(wl.n, rows_n, seed=1)
    Hs = oracle.widen(inp["H"][rows], wl.x_dtype)
    Wx = oracle.widen(inp["W"], wl.x_dtype)
    ids = inp["t_ids"][rows]
    lg = oracle.widen(inp["t_logits"][rows], wl.t_dtype)
    m = None if inp["mask"] is None else inp["mask"][rows]
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max([int(i.get("num_threads", 1)) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.kd_forward(Hs, Wx, ids, lg, m)
    oracle.kd_backward(Hs, Wx, ids, lg, m, want_dw=True)
    dt = time.perf_counter() - t0
    del np
    return {"value": rows.size / dt, "unit": "tokens/s", "cores": cores, "blas": blas, "kind": "oracle",
            "sample": f"{rows.size} seeded positions of {wl.name} (fp64 numpy dense forward + backward "
                      f"incl. their dW contribution), {dt:.1f} s",
            # linear extrapolation (the oracle's cost is per position): not measured
            "extrapolated_full_n_s": round(wl.n * dt / rows.size, 1)}


def vendor_gemm(torch, H, W, rows, kernels, reps=10):
    """The vendor GEMM library (hipBLASLt, through torch.mm) on the GEMM shapes
    of one backward group of `rows` rows, bf16 in and out, next to the fused
    kernel that does the same contraction (per-launch averages of this run).
    Plain products only: no logsumexp, exponentials or teacher terms in the
    projection, bf16 outputs where the fused dH and dW keep fp32 (dW added
    into the fp32 accumulator)."""
    C, D, V = rows, H.shape[1], W.shape[0]
    if C > H.shape[0]:
        return None
    Hc = H[:C]
    g = torch.Generator(device="cuda").manual_seed(1)
    dz = torch.randn(C, V, dtype=torch.bfloat16, device="cuda", generator=g).mul_(1e-5)
    z = torch.empty(C, V, dtype=torch.bfloat16, device="cuda")
    dh = torch.empty(C, D, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(V, D, dtype=torch.bfloat16, device="cuda")
    shapes = {
        "projection Z = H_c W^T (NT)": ("bwd_dz", lambda: torch.mm(Hc, W.t(), out=z)),
        "dH = dZ W (NN)": ("bwd_dh", lambda: torch.mm(dz, W, out=dh)),
        "dW = dZ^T H_c (TN)": ("bwd_dw", lambda: torch.mm(dz.t(), Hc, out=dw)),
    }
    flop = 2.0 * C * D * V
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"library": "hipBLASLt via torch.mm", "rows": C, "reps": reps, "gemms": {}}
    for name, (kind, f) in shapes.items():
        f()
        f()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fused = kernels.get(kind, {}).get("avg_ms")
        res["gemms"][name] = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                              "pct_peak": round(100.0 * flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                              "fused_kernel": kind, "fused_ms": round(fused, 4) if fused else None}
    del dz, z, dh, dw
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    from chunked_kl_loss_row_amd import binding as B
    from chunked_kl_loss_row_amd import inputs
    from chunked_kl_loss_row_amd import loss as L

    torch.cuda.set_device(0)
    wl = inputs.workload(args.workload)
    chunk = args.chunk or wl.chunk
    print(f"[bench] generating {wl.name}: n={wl.n} d={wl.d} v={wl.v} k={wl.k} chunk={chunk}",
          file=sys.stderr, flush=True)
    inp = inputs.make_inputs(wl, seed=0)

    import numpy as np

    def dev(a, tag=None):
        if a is None:
            return None
        if tag == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    if args.copy_mib > 0:
        # plain copy of known size: FETCH_SIZE / WRITE_SIZE of this dispatch over
        # 2^20 * copy_mib bytes is the scale factor of the counters
        x = torch.ones(args.copy_mib * 2 ** 18, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        torch.neg(x, out=y)
        torch.cuda.synchronize()
        del x, y
        torch.cuda.empty_cache()

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    H, W = dev(inp["H"], wl.x_dtype), dev(inp["W"], wl.x_dtype)
    ids, lg = dev(inp["t_ids"]), dev(inp["t_logits"], wl.t_dtype)
    mask = dev(inp["mask"])
    prob = L.make_problem(H, W, ids, lg, chunk, 1.0, args.dw_chunks)
    ws = L.workspace_for(prob, H.device)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    lse = torch.empty(wl.n, dtype=torch.float32, device="cuda")
    dH = torch.empty(wl.n, wl.d, dtype=torch.float32, device="cuda")
    dW = torch.zeros(wl.v, wl.d, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        B.kd_chunked_fwd(prob, H, W, ids, lg, mask, loss, lse, None, None, ws, stream=stream)
        B.kd_chunked_bwd(prob, H, W, ids, lg, mask, lse, None, dH, dW, ws, stream=stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    # the headline steps run with the library's per-kernel event recording off
    B.kd_profile_enable(False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # one event after each step as well (recording an event does not synchronise):
    # per-step times for the median / min next to the mean over the timed region
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        e0.record(stream)
        for i in range(args.steps):
            step()
            marks[i].record(stream)
        e1.record(stream)
        torch.cuda.synchronize()
    sclk = clock.summary()
    power = clock.power_summary()
    junction = clock.temp_summary()
    ms = e0.elapsed_time(e1) / args.steps
    per_step = sorted([e0.elapsed_time(marks[0])] +
                      [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)])
    step_stats = {"median": round(per_step[len(per_step) // 2] if len(per_step) % 2 else
                                  0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2]), 4),
                  "min": round(per_step[0], 4), "max": round(per_step[-1], 4)}
    peak_gib = torch.cuda.max_memory_allocated() / 2 ** 30
    loss_v = float(loss.item())
    # per-kernel durations: a second pass of the same steps with HIP events recorded around every
    # launch on the launch stream (kd_profile.h)
    print(f"[bench] per-kernel pass, {args.steps} steps", file=sys.stderr, flush=True)
    B.kd_profile_enable(True)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(args.steps):
        step()
    p1.record(stream)
    torch.cuda.synchronize()
    kern = B.kd_profile_all()
    B.kd_profile_enable(False)
    profiled_ms = p0.elapsed_time(p1) / args.steps

    N, D, V = wl.n, wl.d, wl.v
    flops_step = 8.0 * N * D * V
    tflops = flops_step / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.x_dtype == "bf16" else PEAK_F32_TFLOPS
    kernels = {k: {"avg_ms": (t / n if n else None), "launches_per_step": n / args.steps,
                   "ms_per_step": t / args.steps} for k, (t, n) in kern.items()}
    # the two stand-alone (memory-bound) passes: algorithmic bytes per step and GB/s
    ts = 2 if wl.t_dtype == "bf16" else 4
    nvt = -(-V // PROJ_TILE_V)
    alg_bytes = {
        # ids + logits + mask read; sorted (key, p), zeroed gather slots, negent, s, tile bounds written
        "prep": 2 * (N * wl.k * (4 + ts) + N + N * wl.k * 12 + N * 8 + N * (nvt + 1) * 2),
        # tile partials (max, sum) + sorted p + gathered z + negent, s, mask read; lse, row loss written
        "merge": N * nvt * 8 + N * wl.k * 8 + N * 9 + N * 12,
    }
    for k, b in alg_bytes.items():
        if k in kernels and kernels[k]["ms_per_step"] > 0:
            kernels[k]["alg_bytes_per_step"] = b
            kernels[k]["GB_s"] = round(b / (kernels[k]["ms_per_step"] * 1e-3) / 1e9, 1)
    dom = max(kern, key=lambda k: kern[k][0])
    roofline = None
    if dom in GEMM_KINDS and kern[dom][1] > 0:
        per_launch_flop = 2.0 * N * D * V / (kern[dom][1] / args.steps)
        avg_s = kern[dom][0] / kern[dom][1] * 1e-3
        ach = per_launch_flop / avg_s / 1e12
        tpath = args.traffic or os.path.join(ROOT, "profiles", f"kd_gemms_{wl.name}_traffic.txt")
        traffic = read_traffic(tpath, dom)
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                    "algorithmic_flop_per_launch": per_launch_flop, "avg_launch_ms": round(avg_s * 1e3, 4)}
        # the rated peak assumes 2.4 GHz; the committed counter summary gives the shader clock this
        # kernel ran at (power-limited): the same achieved rate against the peak at that clock
        clk = read_clock(os.path.join(ROOT, "profiles", f"kd_gemms_{wl.name}_sq_counters.txt"), dom)
        roofline["profiled_clock_ghz"] = clk
        roofline["frac_at_profiled_clock"] = round(ach / (peak * clk / 2.4), 4) if clk else None
        # the same against the peak at the shader clock sampled during this run's timed steps
        # (a step average over all kernels)
        roofline["frac_at_observed_clock"] = round(ach / (peak * sclk["mean"] / 2400.0), 4) if sclk else None

    variants = None
    if not args.no_variants:
        vsteps = max(1, min(args.steps, 5))
        v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # temperature-scaled loss, tau = 2: the same kernels, 1/tau folded into their exponent
        # scales and tau into the dZ coefficients (8 N D V flops, as the headline)
        prob_t = L.make_problem(H, W, ids, lg, chunk, 2.0, args.dw_chunks)

        def step_tau():
            B.kd_chunked_fwd(prob_t, H, W, ids, lg, mask, loss, lse, None, None, ws, stream=stream)
            B.kd_chunked_bwd(prob_t, H, W, ids, lg, mask, lse, None, dH, dW, ws, stream=stream)

        step_tau()
        torch.cuda.synchronize()
        v0.record(stream)
        for _ in range(vsteps):
            step_tau()
        v1.record(stream)
        torch.cuda.synchronize()
        tau_ms = v0.elapsed_time(v1) / vsteps
        variants = {"temperature_2": {
            "entry": f"kd_chunked_fwd + kd_chunked_bwd, tau = 2, dw_chunks = {args.dw_chunks}", "steps": vsteps,
            "ms_per_step": round(tau_ms, 4), "tokens_per_s": round(N / (tau_ms * 1e-3), 1),
            "tflops": round(flops_step / (tau_ms * 1e-3) / 1e12, 2), "loss": float(loss.item())}}

        # the backward chunk by chunk (kd_problem.dw_chunks = 1): one chunk of dZ in the workspace,
        # dW read and written once per chunk; same flops and results as the headline
        other = 1 if args.dw_chunks != 1 else 2
        del ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        prob_g = L.make_problem(H, W, ids, lg, chunk, 1.0, other)
        wsg = L.workspace_for(prob_g, H.device)

        def step_groups():
            B.kd_chunked_fwd(prob_g, H, W, ids, lg, mask, loss, lse, None, None, wsg, stream=stream)
            B.kd_chunked_bwd(prob_g, H, W, ids, lg, mask, lse, None, dH, dW, wsg, stream=stream)

        step_groups()
        torch.cuda.synchronize()
        v0.record(stream)
        for _ in range(vsteps):
            step_groups()
        v1.record(stream)
        torch.cuda.synchronize()
        g_ms = v0.elapsed_time(v1) / vsteps
        variants[f"dw_chunks_{other}"] = {
            "entry": f"kd_chunked_fwd + kd_chunked_bwd, dw_chunks = {other}", "steps": vsteps,
            "ms_per_step": round(g_ms, 4), "tokens_per_s": round(N / (g_ms * 1e-3), 1),
            "tflops": round(flops_step / (g_ms * 1e-3) / 1e12, 2),
            "peak_gib": round(torch.cuda.max_memory_allocated() / 2 ** 30, 3)}
        del wsg

        # kd_chunked_fwd_bwd: the forward keeps each chunk's fp32 logits and dZ is formed from
        # them instead of recomputing the projection (6 N D V flops done; same results bit for bit)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        wsf = torch.empty(B.kd_chunked_fwd_bwd_workspace_size(prob), dtype=torch.uint8, device="cuda")

        def step_single():
            B.kd_chunked_fwd_bwd(prob, H, W, ids, lg, mask, None, loss, lse, dH, dW, wsf, stream=stream)

        step_single()
        torch.cuda.synchronize()
        B.kd_profile_enable(True)
        v0.record(stream)
        for _ in range(vsteps):
            step_single()
        v1.record(stream)
        torch.cuda.synchronize()
        vms = v0.elapsed_time(v1) / vsteps
        vk = B.kd_profile_all()
        B.kd_profile_enable(False)
        variants["single_call_cached_logits"] = {
            "entry": "kd_chunked_fwd_bwd", "steps": vsteps, "ms_per_step": round(vms, 4),
            "tokens_per_s": round(N / (vms * 1e-3), 1),
            "tflops_done": round(6.0 * N * D * V / (vms * 1e-3) / 1e12, 2),
            "peak_gib": round(torch.cuda.max_memory_allocated() / 2 ** 30, 3),
            "kernels": {k: round(t / n, 4) for k, (t, n) in vk.items() if n}}

        # kd_teacher_topk on the same shapes (H, W standing in for a teacher): the K largest
        # logits per row, two projection passes (4 N D V flops done)
        del wsf
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        tprob = B.problem(N, D, V, wl.k, chunk, B.KD_BF16 if wl.x_dtype == "bf16" else B.KD_F32)
        wst = torch.empty(B.kd_teacher_topk_workspace_size(tprob), dtype=torch.uint8, device="cuda")
        tids = torch.empty(N, wl.k, dtype=torch.int32, device="cuda")
        tlog = torch.empty(N, wl.k, dtype=torch.float32, device="cuda")
        ovf = torch.zeros(1, dtype=torch.int32, device="cuda")

        def step_topk():
            B.kd_teacher_topk(tprob, H, W, tids, tlog, ovf, wst, stream=stream)

        step_topk()
        torch.cuda.synchronize()
        B.kd_profile_enable(True)
        v0.record(stream)
        for _ in range(vsteps):
            step_topk()
        v1.record(stream)
        torch.cuda.synchronize()
        tms = v0.elapsed_time(v1) / vsteps
        tk = B.kd_profile_all()
        B.kd_profile_enable(False)
        variants["teacher_topk_producer"] = {
            "entry": "kd_teacher_topk", "k": wl.k, "steps": vsteps, "ms_per_pass": round(tms, 4),
            "tokens_per_s": round(N / (tms * 1e-3), 1),
            "tflops_done": round(4.0 * N * D * V / (tms * 1e-3) / 1e12, 2),
            "overflow_rows": int(ovf.item()),
            "kernels": {k: round(t / n, 4) for k, (t, n) in tk.items() if n}}
        del wst

    vendor = None
    if args.vendor_gemm and wl.x_dtype == "bf16":
        vendor = vendor_gemm(torch, H, W, args.dw_chunks * chunk, kernels)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu oracle baseline on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, args.cpu_rows)

    out = {
        "metric": METRIC,
        "value": round(N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.x_dtype,
        "data": "synthetic (seeded; shapes and value recipe of the workload)",
        "config": {"workload": wl.name, "n": N, "d": D, "v": V, "k": wl.k, "chunk": chunk,
                   "dw_chunks": args.dw_chunks, "mask": wl.mask, "ids": wl.ids, "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2),
        "pct_peak": round(100.0 * tflops / peak, 2),
        # shader clock sampled during the timed steps (MHz; the rated peak assumes 2400) and the
        # step's rate against the peak at that clock
        "observed_sclk_mhz": sclk,
        "pct_peak_at_observed_clock": round(100.0 * tflops / (peak * sclk["mean"] / 2400.0), 2) if sclk else None,
        # board power and junction temperature sampled over the same steps (null where the card's
        # hwmon entries are missing): at this load the chip sits at its power cap
        "observed_power_w": power,
        "observed_junction_c": junction,
        "peak_gib": round(peak_gib, 3),
        "profiled_ms_per_step": round(profiled_ms, 4),
        "loss": loss_v,
        "roofline": roofline,
        "kernels": kernels,
        "variants": variants,
        "vendor_gemm": vendor,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
