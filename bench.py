"""Benchmark of the Sketch Attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

A step is one full forward (the streaming kernel and the merge) over one
batch of synthetic histories already resident in HBM: by default the full
100K workload (B=16 users x L=100,000 rows, H=8 heads, m=128 prototypes,
dh=64, bf16, packed with int32 offsets).  Prints ONE JSON line with the
whole-job throughput in history tokens per second, the roofline of the
streaming kernel (algorithmic bytes / its HIP-event-timed duration against
the 8 TB/s HBM peak) and the CPU oracle timed on a bounded sample on this
host as a baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "history tokens/sec compressed by SA (bf16, 100K varlen) + % HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_full100k_bf16.json")


class _Hip:
    """Just enough of the HIP runtime (via ctypes) for timing events."""

    def __init__(self):
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                self.lib = ctypes.CDLL(name)
                break
            except OSError:
                continue
        else:
            raise RuntimeError("libamdhip64.so not found")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def _percentiles(xs):
    """10th, 50th and 90th percentile of a list of launch times (nearest rank)."""
    ys = sorted(xs)
    return [ys[min(len(ys) - 1, int(q * len(ys)))] for q in (0.1, 0.5, 0.9)]


def _kernel_hash(kernel: str = "sa_bf16_stream_kernel") -> str:
    from sketch_attention_flashsa_amd.build import KERNEL_SOURCES, sources_hash
    return sources_hash(KERNEL_SOURCES.get(kernel))


def _traffic(kernel: str):
    """HBM bytes per launch of the streaming kernel from the committed
    rocprofv3 counter summary, or None if absent, taken on another kernel or
    on other sources."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256_16") != _kernel_hash(kernel) or t.get("kernel") != kernel:
        return None
    return t.get("hbm_bytes_per_launch")


def copy_calibration(mib: int, steps: int) -> None:
    """A plain elementwise copy (torch.neg, bf16) that reads and writes
    mib MiB per launch: the reference for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"calibration": "copy", "kernel": "neg (elementwise)", "bytes_read": 2 * n,
                      "bytes_written": 2 * n, "launches": steps, "ms_per_launch": dt * 1e3,
                      "GBps": 4 * n / dt / 1e9}))


def hbm_probe(mib: int, steps: int) -> None:
    """Plain torch kernels over an fp32 buffer of mib MiB, timed with events
    after a warm-up: a fill (write only), a sum (read only) and a copy_ (read
    and write).  The rates bound what a kernel with the same read/write mix
    can reach on this device."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    out = {"probe": "hbm", "bytes": 4 * n}
    for name, fn, nbytes in (("fill", lambda: y.fill_(1.0), 4 * n), ("sum", lambda: x.sum(), 4 * n),
                             ("copy", lambda: y.copy_(x), 8 * n)):
        for _ in range(10):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        out[name] = {"ms": ms, "GBps": nbytes / ms / 1e6}
    print(json.dumps(out))


def device_reference(mib: int = 2048, read_iters: int = 400, copy_iters: int = 150, gemm_n: int = 8192,
                     gemm_iters: int = 60, timed: int = 40):
    """The device's own rates, measured in this process just before the
    benchmark's warm-up, with torch's kernels: a sum over an fp32 buffer of
    `mib` MiB (reads only), its copy_ into a second buffer (reads and
    writes) and a dense bf16 GEMM of size gemm_n^3 (the vendor BLAS), each
    run back to back with the last `timed` launches timed by events.  The
    streaming kernel is compared with these two torch kernels' rates as well
    as with the nominal 8 TB/s; they are what torch's own kernels reach on
    the device, not its bandwidth ceiling (torch's sum, a reduction, stays
    near 4 TB/s).  The ~0.4 s of work, the last part of it at the
    board's power limit, also brings the chip from idle into the loaded power
    state that the timed steps run in: after idle, the power controller lets
    the first launches run at full clock, then cuts the clock hard for a few
    tens of launches before it settles (the `from_idle` object of the result
    line shows that transient for the same launches)."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    ga = torch.randn(gemm_n, gemm_n, dtype=torch.bfloat16, device="cuda:0")
    gb = torch.randn(gemm_n, gemm_n, dtype=torch.bfloat16, device="cuda:0")
    out = {"buffer_mib": mib, "gemm_n": gemm_n}
    for name, fn, iters, nbytes in (("torch_sum", lambda: x.sum(), read_iters, 4 * n),
                                    ("torch_copy", lambda: y.copy_(x), copy_iters, 8 * n),
                                    ("gemm", lambda: ga @ gb, gemm_iters, 0)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(iters):
            if i == iters - timed:
                a.record()
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / timed
        if nbytes:
            out[f"{name}_GBps"] = nbytes / ms / 1e6
        else:
            out["gemm_bf16_TFLOPs"] = 2.0 * gemm_n ** 3 / ms / 1e9
    del x, y, ga, gb
    return out


def from_idle(step, steps: int, warmup: int, idle_s: float = 1.0):
    """The same warm-up and timed launches after `idle_s` seconds of idle
    device: per-launch durations of the streaming kernel (HIP events), the
    power-management transient that the reference work above removes."""
    import torch
    import sketch_attention_flashsa_amd as sa
    hip = _Hip()
    torch.cuda.synchronize()
    time.sleep(idle_s)
    n = warmup + steps
    evs = [(hip.event(), hip.event()) for _ in range(n)]
    for i in range(n):
        sa.sa_set_timing_events(evs[i][0], evs[i][1])
        step()
    torch.cuda.synchronize()
    ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    timed = ms[warmup:]
    return {"idle_s": idle_s, "kernel_ms_first_launches": [round(x, 4) for x in ms[:min(n, 30)]],
            "kernel_ms_avg_timed_launches": sum(timed) / len(timed)}


def cpu_baseline(w, n_users: int):
    """The oracle as it stands, on the first n_users users of the workload."""
    import oracle
    n = min(n_users, w["B"])
    if w["layout"] == "packed":
        cu = w["cu_offsets"][: n + 1].clone()
        rows = int(cu[-1])
        t0 = time.perf_counter()
        oracle.forward(w["P"], w["K"][:rows], w["V"][:rows], cu_offsets=cu)
    else:
        rows = int(w["lengths"][:n].sum())
        t0 = time.perf_counter()
        oracle.forward(w["P"], w["K"][:n], w["V"][:n], lengths=w["lengths"][:n])
    dt = time.perf_counter() - t0
    pairs = n * w["H"]
    return {
        "value": rows / dt,
        "unit": "tokens/s",
        # OpenMP threads the oracle ran (its loop has n * H iterations)
        "cores": int(min(oracle.threads(), pairs)),
        "host_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"first {n} users of the workload ({rows} history rows, all {w['H']} heads and {w['m']} "
                  f"prototypes), double precision, {dt:.1f} s wall",
    }


_REF = {}


def _preconditioned(args, step):
    """The timed region of the secondary legs: the device reference work of
    the main leg first (which also brings the chip out of its post-idle clock
    transient), then `_timed`.  The reference rates go into the result line."""
    _REF.clear()
    if getattr(args, "ref_mib", 0) > 0:
        _REF.update(device_reference(args.ref_mib))
    return _timed(step, args.steps, args.warmup)


def _emit(out: dict) -> None:
    if _REF:
        out["device_reference"] = dict(_REF)
    print(json.dumps(out))


def _power_file():
    """The board power reading of the one visible GPU (amdgpu hwmon
    power1_input, microwatts) and its cap, or (None, None)."""
    import glob
    found = []
    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        try:
            with open(os.path.join(d, "name")) as fh:
                if fh.read().strip() != "amdgpu":
                    continue
            with open(os.path.join(d, "power1_input")) as fh:
                int(fh.read())
        except (OSError, ValueError):
            continue
        cap = None
        try:
            with open(os.path.join(d, "power1_cap")) as fh:
                cap = int(fh.read()) / 1e6
        except (OSError, ValueError):
            pass
        found.append((os.path.join(d, "power1_input"), cap))
    return found[0] if len(found) == 1 else (None, None)


def power_leg(step, seconds: float):
    """Back-to-back steps for ``seconds`` while a thread reads the board's
    power every 5 ms: the loaded power (against the board's cap) and the
    kernel's event-timed duration under it.  None without a readable power
    file (or with several GPUs' files, which would be ambiguous)."""
    import threading
    import torch
    import sketch_attention_flashsa_amd as sa
    path, cap = _power_file()
    if path is None or seconds <= 0:
        return None
    hip = _Hip()
    watts, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                with open(path) as fh:
                    watts.append(int(fh.read()) / 1e6)
            except (OSError, ValueError):
                pass
            time.sleep(0.005)

    th = threading.Thread(target=sample, daemon=True)
    kern = []
    evs = [(hip.event(), hip.event()) for _ in range(8)]
    n = 0
    t0 = time.perf_counter()
    th.start()
    try:
        while time.perf_counter() - t0 < seconds:
            # launches in batches of 64 (events on 8 of them), so the queue
            # stays short; the chip never idles between batches for long
            for i in range(64):
                if i % 8 == 0:
                    a, b = evs[i // 8]
                    sa.sa_set_timing_events(a, b)
                step()
            torch.cuda.synchronize()
            kern.extend(hip.elapsed_ms(a, b) for a, b in evs)
            n += 64
    finally:
        stop.set()
        th.join()
        for a, b in evs:
            hip.destroy(a)
            hip.destroy(b)
    dt = time.perf_counter() - t0
    # the first 0.5 s of samples cover the ramp to the loaded state
    tail = [w for i, w in enumerate(watts) if i * 0.005 >= 0.5] or watts
    return {"seconds": round(dt, 3), "steps": n, "board_power_w_avg": sum(tail) / len(tail) if tail else None,
            "board_power_w_max": max(watts) if watts else None, "power_cap_w": cap, "power_samples": len(watts),
            "kernel_ms_avg": sum(kern) / len(kern), "kernel_ms_p10_p50_p90": _percentiles(kern)}


def _timed(step, steps: int, warmup: int, flush_mib: int = 0, flush_kind: str = "write"):
    """Run warmup + timed steps; returns (ms per step, the streaming kernel's
    HIP-event durations in ms).  ms per step is the wall clock over the timed
    loop; with flush_mib > 0 a buffer of that size is overwritten before every
    step (so no input is left in the L2 or the 256 MB MALL; flush_kind "read"
    sums it instead) and ms per step is the mean of per-step event times,
    which exclude the flush."""
    import torch
    import sketch_attention_flashsa_amd as sa
    hip = _Hip()
    scratch = torch.ones(flush_mib << 18, dtype=torch.float32, device="cuda:0") if flush_mib > 0 else None

    def flush():
        if flush_kind == "read":
            scratch.sum()
        else:
            scratch.fill_(1.0)

    for _ in range(warmup):
        if scratch is not None:
            flush()
        step()
    torch.cuda.synchronize()
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(steps if scratch is not None else 0)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            flush()
            step_evs[i][0].record()
        sa.sa_set_timing_events(evs[i][0], evs[i][1])
        step()
        if scratch is not None:
            step_evs[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    if scratch is not None:
        return sum(a.elapsed_time(b) for a, b in step_evs) / steps, kern_ms
    return (t1 - t0) * 1e3 / steps, kern_ms


def bench_fused(args, w):
    """The fused-projection workload: X [rows, d_model] and Wk, Wv resident in
    HBM; the fused kernel is bounded by MFMA (and the softmax exps)."""
    import torch
    import workloads as W
    import sketch_attention_flashsa_amd as sa
    from sketch_attention_flashsa_amd import flops
    dev = torch.device("cuda:0")
    spec = w["spec"]
    B, H, m, dh, dm = w["B"], w["H"], w["m"], w["dh"], w["d_model"]
    tokens = int(w["lengths"].sum())
    X, Wk, Wv, P = (w[k].to(dev) for k in ("X", "Wk", "Wv", "P"))
    cu = w["cu_offsets"].to(dev)
    S = torch.empty((B, H, m, dh), dtype=torch.float32, device=dev)
    pb = sa.make_problem(B, H, m, dh, X.shape[0], dtype="bf16")
    ws = torch.empty(sa.load_library().sa_forward_fused_proj_workspace_size(ctypes.byref(pb), dm),
                     dtype=torch.uint8, device=dev)

    def step():
        sa.sa_forward_fused_proj(X, Wk, Wv, P, cu, out=S, workspace=ws)

    ms_per_step, kern_ms = _preconditioned(args, step)
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    fl = flops.sa_forward_flops(tokens, H, m, dh) + flops.projection_flops(tokens, dm, H * dh, 2)
    tflops = fl / (kern_avg_ms / 1e3) / 1e12
    alg_bytes = tokens * dm * 2 + 2 * dm * H * dh * 2 + H * m * dh * 2 + 4 * (B + 1)
    exps = tokens * H * m
    out = {
        "metric": METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws shaped like the paper's histories)",
        "config": {"workload": spec.name, "B": B, "sum_L": tokens, "L_max": int(w["lengths"].max()), "H": H,
                   "m": m, "dh": dh, "d_model": dm, "layout": "packed", "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "sa_fused_proj_kernel",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": fl,
            "kernel_ms_avg": kern_avg_ms,
            "kernel_ms_min": min(kern_ms),
            "hbm_GBps": alg_bytes / (kern_avg_ms / 1e3) / 1e9,
            "exp_per_s": exps / (kern_avg_ms / 1e3),
        },
        "cpu_baseline": None,
    }
    _emit(out)


REFINE_METRIC = "history tokens/sec through stacked SA refinement (bf16, 2 layers, fused-workload shape)"


def bench_refine(args):
    """Stacked refinement (two layers, the paper's N_sa = 2) over the fused
    workload's users: each layer's attention pass streams X with the keys
    projected on chip, then the sketch update (layer norms, SwiGLU FFN, next
    queries) runs on MFMA.  Timed end to end (every launch of the call)."""
    import torch
    import workloads as W
    import sketch_attention_flashsa_amd as sa
    from sketch_attention_flashsa_amd import flops
    dev = torch.device("cuda:0")
    w = W.make(5)
    B, H, m, dh, dm = w["B"], w["H"], w["m"], w["dh"], w["d_model"]
    n_layers = 2
    tokens = int(w["lengths"].sum())
    X, cu = w["X"].to(dev), w["cu_offsets"].to(dev)
    P0 = W.random_refine_case(6, B=1, H=H, m=m, dh=dh, lengths=[1])["P0"].to(dev)
    layers = [{k: v.to(dev) for k, v in L.items()} for L in W.refine_layers(6, dm, n_layers)]
    out = torch.empty((B, m, dm), dtype=torch.float32, device=dev)
    pb = sa.make_problem(B, H, m, dh, X.shape[0], dtype="bf16")
    ws = torch.empty(sa.sa_refine_workspace_size(pb, dm, n_layers), dtype=torch.uint8, device=dev)

    def step():
        sa.sa_refine_forward(X, P0, layers, cu, H, out=out, workspace=ws)

    ms_per_step, call_ms = _preconditioned(args, step)
    call_avg = sum(call_ms) / len(call_ms)
    fl = flops.refine_flops(tokens, B, m, dm, n_layers)
    tflops = fl / (call_avg / 1e3) / 1e12
    _emit(({
        "metric": REFINE_METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws shaped like the paper's histories; random-init layers)",
        "config": {"workload": "refine2_fusedproj_bf16", "B": B, "sum_L": tokens, "L_max": int(w["lengths"].max()),
                   "H": H, "m": m, "dh": dh, "d_model": dm, "n_layers": n_layers, "layout": "packed",
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "sa_refine_forward (all launches of one call)",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": fl,
            "kernel_ms_avg": call_avg,
            "kernel_ms_min": min(call_ms),
        },
        "cpu_baseline": None,
    }))


BACKWARD_METRIC = "history tokens/sec through the SA backward pass (bf16, 100K varlen) + % HBM peak"


def bench_backward(args):
    """The backward pass on the 100K workload: S, lse from one forward and a
    seeded upstream gradient dS are resident; a step is one sa_backward call
    (all of its launches, bracketed by the timing events)."""
    import numpy as np
    import torch
    import workloads as W
    import sketch_attention_flashsa_amd as sa
    from sketch_attention_flashsa_amd import flops
    dev = torch.device("cuda:0")
    w = W.make(4)
    B, H, m, dh = w["B"], w["H"], w["m"], w["dh"]
    tokens = int(w["lengths"].sum())
    P, K, V, cu = (w[k].to(dev) for k in ("P", "K", "V", "cu_offsets"))
    mask = None
    if args.mask_p > 0:
        keep = np.random.default_rng(77).uniform(size=K.shape[0]) >= args.mask_p
        mask = torch.from_numpy(keep.astype(np.uint8)).to(dev)
    S, lse = sa.sa_forward(P, K, V, cu_offsets=cu, mask=mask, return_lse=True)
    dS = torch.from_numpy(np.random.default_rng(8).standard_normal((B, H, m, dh), dtype=np.float32)).to(dev)
    pb = sa.make_problem(B, H, m, dh, K.shape[0], dtype="bf16")
    ws = torch.empty(sa.sa_backward_workspace_size(pb), dtype=torch.uint8, device=dev)
    gdt = torch.bfloat16 if args.grad_dtype == "bf16" else torch.float32
    gsz = 2 if args.grad_dtype == "bf16" else 4
    out = (torch.empty(P.shape, dtype=torch.float32, device=dev), torch.zeros(K.shape, dtype=gdt, device=dev),
           torch.zeros(V.shape, dtype=gdt, device=dev))

    def step():
        sa.sa_backward(P, K, V, S, lse, dS, cu_offsets=cu, mask=mask, workspace=ws, out=out)

    ms_per_step, call_ms = _preconditioned(args, step)
    call_avg = sum(call_ms) / len(call_ms)
    # every K, V element read once, dK, dV written once (fp32 or bf16), plus P, dP, S, dS, lse and offsets
    alg_bytes = tokens * H * dh * (2 + 2 + 2 * gsz) + H * m * dh * (2 + 4) + B * H * m * (dh * 8 + 4) + 4 * (B + 1)
    achieved = alg_bytes / (call_avg / 1e3) / 1e9
    _emit(({
        "metric": BACKWARD_METRIC + (", bf16 gradients" if args.grad_dtype == "bf16" else "")
        + (", masked rows" if mask is not None else ""),
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws shaped like the paper's histories)",
        "config": {"workload": "backward_full100k_bf16", "B": B, "sum_L": tokens, "L_max": int(w["lengths"].max()),
                   "H": H, "m": m, "dh": dh, "layout": "packed", "grad_dtype": args.grad_dtype, "mask_p": args.mask_p,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "sa_backward (all launches of one call)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes_per_launch": alg_bytes,
            "kernel_ms_avg": call_avg,
            "kernel_ms_min": min(call_ms),
            "mfma_tflops": 2.5 * flops.sa_forward_flops(tokens, H, m, dh) / (call_avg / 1e3) / 1e12,
        },
        "cpu_baseline": None,
    }))


PRODUCTION_METRIC = "history tokens/sec through SA at the paper's production shape (bf16, d=128, k=1024, V=X)"


def bench_production(args):
    """The paper's production SA shape (appendix G.5: one head of width 128,
    1024 prototypes, values = X, keys X W_K) over 16 users of 100,000 rows,
    through the fused entry: W_K folded into the prototypes once per call
    (the scores P (X W_K)^T are (P W_K^T) X^T, so K is never formed), then the
    streaming forward over X.  Bounded by MFMA.  The roofline counts the
    FLOPs performed (the fold and the two products per row); the original
    formulation's count, with the per-row key projection, is reported beside
    it."""
    import numpy as np
    import torch
    import workloads as W
    import sketch_attention_flashsa_amd as sa
    from sketch_attention_flashsa_amd import flops
    dev = torch.device("cuda:0")
    B, L, H, m, dh, dm = 16, 100_000, 1, 1024, 128, 128
    w = W.random_fused_case(8, B=1, H=H, m=m, dh=dh, d_model=dm, lengths=[1], w_var=1.0 / dm)
    g = torch.Generator().manual_seed(8)
    X = torch.randn(B * L, dm, generator=g).to(torch.bfloat16).to(dev)
    Wk, P = w["Wk"].to(dev), w["P"].to(dev)
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device=dev)
    tokens = B * L
    S = torch.empty((B, H, m, dh), dtype=torch.float32, device=dev)
    pb = sa.make_problem(B, H, m, dh, tokens, dtype="bf16")
    ws = torch.empty(sa.load_library().sa_forward_fused_proj_workspace_size(ctypes.byref(pb), dm),
                     dtype=torch.uint8, device=dev)

    def step():
        sa.sa_forward_fused_proj(X, Wk, None, P, cu, out=S, workspace=ws)

    ms_per_step, call_ms = _preconditioned(args, step)
    call_avg = sum(call_ms) / len(call_ms)
    fl = flops.sa_forward_flops(tokens, H, m, dh) + flops.fold_keys_flops(H, m, dh, dm)
    fl_orig = flops.sa_forward_flops(tokens, H, m, dh) + flops.projection_flops(tokens, dm, H * dh, 1)
    tflops = fl / (call_avg / 1e3) / 1e12
    _emit(({
        "metric": PRODUCTION_METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws; random-init projection)",
        "config": {"workload": "production_d128_k1024_bf16", "B": B, "sum_L": tokens, "L_max": L, "H": H, "m": m,
                   "dh": dh, "d_model": dm, "layout": "packed", "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "prototype fold + sa_bf16_stream_d128_kernel + merge",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": fl,
            "original_formulation_flops_per_launch": fl_orig,
            "original_formulation_tflops": fl_orig / (call_avg / 1e3) / 1e12,
            "kernel_ms_avg": call_avg,
            "kernel_ms_min": min(call_ms),
            "exp_per_s": tokens * H * m / (call_avg / 1e3),
        },
        "cpu_baseline": None,
    }))


STCA_METRIC = "targets/sec through STCA single-query attention, reordered (bf16, D=1024, h=16)"


def bench_stca(args):
    """STCA single-query attention (appendix G.2.1's reordering) over the
    sketch branch: 64 users, each a sketch of 1,024 rows adapted to width
    D = 1024 and 40 targets (the training-side reuse ratio of appendix G.5),
    h = 16 heads.  A step is one sa_stca_attention call; the roofline covers
    its launches after the weight transpose (MFMA-bound), timed by the HIP
    events the library records around them."""
    import numpy as np
    import torch
    import workloads as W
    import sketch_attention_flashsa_amd as sa
    from sketch_attention_flashsa_amd import flops
    dev = torch.device("cuda:0")
    B, L, R, D, h = 64, args.stca_rows, args.stca_targets, 1024, 16
    w = W.random_stca_case(9, lengths=[L] * B, targets=[R] * B, D=D, h=h)
    xt, X, Wq, Wk, Wv, cu, toff = (w[k].to(dev) for k in ("xt", "X", "Wq", "Wk", "Wv", "cu_offsets", "t_offsets"))
    T = w["T"]
    pb = sa.SaStcaProblem(B=B, T=T, D=D, h=h, total_rows=B * L, x_row_stride=0, scale=0.0, flags=0)
    ws = torch.empty(sa.sa_stca_workspace_size(pb), dtype=torch.uint8, device=dev)
    out = torch.empty((T, D), dtype=torch.float32, device=dev)

    def step():
        sa.sa_stca_attention(xt, X, Wq, Wk, Wv, cu, toff, h, workspace=ws, out=out)

    ms_per_step, kern_ms = _preconditioned(args, step)
    kavg = sum(kern_ms) / len(kern_ms)
    fl = flops.stca_attention_flops([L] * T, D, h)
    tflops = fl / (kavg / 1e3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        from oracle import stca as ST
        nu = min(B, 32)
        n = nu * R
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        t0 = time.perf_counter()
        ST.stca_attention(w["xt"][:n], w["X"][:nu * L], w["Wq"], w["Wk"], w["Wv"], w["cu_offsets"][:nu + 1].numpy(),
                          w["t_offsets"][:nu + 1].numpy(), h)
        dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "targets/s", "cores": int(blas), "kind": "oracle",
               "sample": f"the first {nu} users ({n} targets, {L} rows each, all {h} heads), double precision, "
                         f"{dt:.1f} s wall"}
    _emit(({
        "metric": STCA_METRIC,
        "value": T / (ms_per_step / 1e3),
        "unit": "targets/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws; random-init projections)",
        "config": {"workload": f"stca_sketch_L{L}_R{R}_bf16", "B": B, "rows_per_user": L, "targets_per_user": R,
                   "D": D, "h": h, "dh": D // h, "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "sa_stca_attention: query GEMM + sa_stca_kernel<1024, 64> + output GEMM",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": fl,
            "kernel_ms_avg": kavg,
            "kernel_ms_min": min(kern_ms),
        },
        "cpu_baseline": cpu,
    }))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The device lowers its clocks for a few tens of back-to-back launches
    # before it settles; 50 untimed steps (~40 ms) keep that out of the timing.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=4,
                    help="workload number (default 4: full 100K bf16; 5: fused projection; 6: two refinement "
                         "layers; 7: backward pass on the 100K workload; 8: production shape d=128, k=1024; "
                         "9: STCA single-query attention over the sketch)")
    ap.add_argument("--stca-rows", type=int, default=1024, help="workload 9: rows per user (1024: the sketch)")
    ap.add_argument("--stca-targets", type=int, default=40, help="workload 9: targets per user")
    ap.add_argument("--norm", choices=("history", "prototype"), default="history",
                    help="workloads 1-4: softmax axis (prototype = the paper's normalisation display, row A9)")
    ap.add_argument("--mask-p", type=float, default=0.0,
                    help="workloads 1-4 and 7: pass a seeded per-row mask that excludes each row with this probability")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="workloads 1-4: overwrite a buffer of this many MiB before every step (cold caches)")
    ap.add_argument("--flush-kind", choices=("write", "read"), default="write",
                    help="--flush-mib: overwrite (write) or sum (read) the buffer before each step")
    ap.add_argument("--cold-mib", type=int, default=1024,
                    help="workloads 1-4: after the timed steps, time the kernel again with this many MiB "
                         "overwritten before each launch (0: skip); reported as cold_cache")
    ap.add_argument("--grad-dtype", choices=("fp32", "bf16"), default="fp32",
                    help="workload 7: element type of dK and dV")
    ap.add_argument("--cpu-users", type=int, default=4, help="users in the CPU oracle sample")
    ap.add_argument("--power-s", type=float, default=2.0,
                    help="workloads 1-4: after the timed steps, this many seconds of back-to-back steps with the "
                         "board power read every 5 ms (0: skip); reported as sustained_power")
    ap.add_argument("--dense-lengths", action="store_true",
                    help="dense workloads: pass the per-user lengths even when all equal the slot size "
                         "(adds the kernel that places users on the virtual row axis)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ref-mib", type=int, default=2048,
                    help="workloads 1-4: before the warm-up, measure the device's read and copy rates over a "
                         "buffer of this many MiB and its dense bf16 GEMM rate (0: skip); reported as "
                         "device_reference")
    ap.add_argument("--no-from-idle", dest="from_idle", action="store_false",
                    help="workloads 1-4: skip the launches timed after an idle second (from_idle)")
    ap.add_argument("--hbm-probe-mib", type=int, default=0,
                    help="time torch fill / sum / copy_ over a buffer of this many MiB and exit")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the forward, time a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the forward has no multi-GPU path in this build "
              "(users shard across GPUs with no exchange; run one process per GPU).", file=sys.stderr)
        sys.exit(2)

    if args.hbm_probe_mib:
        hbm_probe(args.hbm_probe_mib, args.steps)
        return
    if args.copy_mib:
        copy_calibration(args.copy_mib, args.steps)
        return

    import torch
    import workloads as W
    import sketch_attention_flashsa_amd as sa
    from sketch_attention_flashsa_amd import flops

    if args.workload == 6:
        return bench_refine(args)
    if args.workload == 7:
        return bench_backward(args)
    if args.workload == 8:
        return bench_production(args)
    if args.workload == 9:
        return bench_stca(args)
    dev = torch.device("cuda:0")
    w = W.make(args.workload)
    spec = w["spec"]
    B, H, m, dh = w["B"], w["H"], w["m"], w["dh"]
    tokens = int(w["lengths"].sum())
    if "X" in w:
        return bench_fused(args, w)
    P, K, V = w["P"].to(dev), w["K"].to(dev), w["V"].to(dev)
    mask = None
    if args.mask_p > 0:
        # seeded per-row mask over the K/V buffer rows: each row excluded with probability mask_p
        import numpy as np
        nrow = K.shape[0] if w["layout"] == "packed" else K.shape[0] * K.shape[1]
        keep = np.random.default_rng(77).uniform(size=nrow) >= args.mask_p
        mask = torch.from_numpy(keep.astype(np.uint8)).to(dev)
    cu = w["cu_offsets"].to(dev) if w["layout"] == "packed" else None
    # dense layout: per-user lengths only when some user is shorter than the
    # slot (with every length equal to L_max the slot is the whole history)
    dense_short = w["layout"] == "dense" and int(w["lengths"].min()) < K.shape[1]
    lengths = w["lengths"].to(dev) if dense_short or (w["layout"] == "dense" and args.dense_lengths) else None
    S = torch.empty((B, H, m, dh), dtype=torch.float32, device=dev)
    pb_kw = {"norm": args.norm}
    proto = args.norm == "prototype"
    # one workspace for all steps (no allocation inside the timed region)
    rows = K.shape[0] if cu is not None else B * K.shape[1]
    pb = sa.make_problem(B, H, m, dh, rows, L_max=0 if cu is not None else K.shape[1], dtype=w["dtype"],
                         norm=args.norm)
    ws = torch.empty(sa.sa_forward_workspace_size(pb), dtype=torch.uint8, device=dev)
    kernel = sa.sa_forward_kernel_name(pb)

    def step():
        sa.sa_forward(P, K, V, cu_offsets=cu, lengths=lengths, mask=mask, out=S, workspace=ws, **pb_kw)

    idle = from_idle(step, args.steps, args.warmup) if args.from_idle else None
    ref = device_reference(args.ref_mib) if args.ref_mib > 0 else None
    ms_per_step, kern_ms = _timed(step, args.steps, args.warmup, args.flush_mib, args.flush_kind)
    value = tokens / (ms_per_step / 1e3)
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    # shapes the one-pass prototype-axis kernel does not serve add a per-row
    # log-sum-exp pass over K before the streaming kernel: their roofline
    # covers the whole call
    two_pass = proto and kernel != "sa_proto_stream_kernel"
    if two_pass:
        kern_ms = [ms_per_step]
        kern_avg_ms = ms_per_step
        kernel = "sa_forward, prototype axis (row log-sum-exp pass + " + kernel + " + merge)"
    el = 2 if w["dtype"] == "bf16" else 4
    # algorithmic bytes of the streaming kernel: every K and V element once, plus P and offsets
    alg_bytes = 2 * tokens * H * dh * el + H * m * dh * el + 4 * (B + 1) + (tokens if mask is not None else 0)
    achieved = alg_bytes / (kern_avg_ms / 1e3) / 1e9
    step_bytes = W.algorithmic_bytes(w)
    out = {
        "metric": METRIC + (", prototype axis" if proto else "") + (", masked rows" if mask is not None else ""),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded normal draws shaped like the paper's histories)",
        "config": {"workload": spec.name, "B": B, "sum_L": tokens, "L_max": int(w["lengths"].max()), "H": H,
                   "m": m, "dh": dh, "layout": w["layout"] + ("+lengths" if lengths is not None else ""),
                   "mask_p": args.mask_p, "flush_mib": args.flush_mib,
                   "flush_kind": args.flush_kind if args.flush_mib else None,
                   "parallelism": "single GPU"},
        "hbm_frac_step": step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": _traffic(kernel) if spec.name == "full100k_bf16" and not proto and mask is None else None,
            "algorithmic_bytes_per_launch": alg_bytes,
            "kernel_ms_avg": kern_avg_ms,
            "kernel_ms_min": min(kern_ms),
            "kernel_ms_p10_p50_p90": _percentiles(kern_ms),
            "mfma_tflops": flops.sa_forward_flops(tokens, H, m, dh) / (kern_avg_ms / 1e3) / 1e12,
        },
        "cpu_baseline": None,
    }
    if ref is not None:
        out["device_reference"] = ref
        out["roofline"]["frac_of_torch_sum"] = achieved / ref["torch_sum_GBps"]
        out["roofline"]["frac_of_torch_copy"] = achieved / ref["torch_copy_GBps"]
    if idle is not None:
        idle["frac"] = alg_bytes / (idle["kernel_ms_avg_timed_launches"] / 1e3) / 1e9 / HBM_PEAK_GBS
        out["from_idle"] = idle
    if args.flush_mib == 0 and args.power_s > 0 and not two_pass:
        pw = power_leg(step, args.power_s)
        if pw is not None:
            pw["frac"] = alg_bytes / (pw["kernel_ms_avg"] / 1e3) / 1e9 / HBM_PEAK_GBS
            out["sustained_power"] = pw
    if args.flush_mib == 0 and args.cold_mib > 0 and not two_pass:
        # the same launches with a buffer overwritten before each one (after
        # the timed region above, which it does not affect): no input left in
        # the L2 or the MALL, and the kernel not launched back to back
        _, cold_ms = _timed(step, args.steps, args.warmup, args.cold_mib)
        cold_avg = sum(cold_ms) / len(cold_ms)
        out["cold_cache"] = {"flush_mib": args.cold_mib, "kernel_ms_avg": cold_avg,
                             "kernel_ms_p10_p50_p90": _percentiles(cold_ms),
                             "achieved": alg_bytes / (cold_avg / 1e3) / 1e9,
                             "frac": alg_bytes / (cold_avg / 1e3) / 1e9 / HBM_PEAK_GBS}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_users)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
