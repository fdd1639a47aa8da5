#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

A step is one fused causal forward over [B=1, H=32, N=16384, d=128] bf16 (the
pages' 16K-token example), inputs resident in HBM before the timed region.
The headline runs exactly the given warm-up steps; each other record also
warms up for 0.25 s of back-to-back calls.
value = algorithmic attention TFLOP/s = 4·d·pairs·B·H / time, pairs = N(N+1)/2.
The same JSON line also carries the other configurations of the hot path
(32K and non-causal forward, the recomputing backward, paged decode in GB/s),
the roofline of the dominant kernel and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only fwd|bwd|decode|...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (fwd/bwd, % bf16 MFMA peak); paged-decode GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
KERNEL_SOURCES = {          # sources a kernel's counters depend on
    "fwd_w64_kernel": ["exact_attention_fwd_amd/csrc/fa_fwd.hip", "exact_attention_fwd_amd/csrc/fa_device.h"],
    "decode_split_kernel": ["exact_attention_fwd_amd/csrc/fa_decode.hip", "exact_attention_fwd_amd/csrc/fa_device.h"],
}


def fwd_kernel_name(d, paged=False, rope=False):
    """The forward kernel a launch runs: 64-query wavefronts for dense d = 128,
    the 32-query kernel otherwise."""
    return "fwd_w64_kernel" if (d == 128 and not paged and not rope) else "fwd_bf16_kernel"


def pairs(N, causal):
    return N * (N + 1) // 2 if causal else N * N


def fwd_flops(B, H, N, d, causal):
    return 4.0 * d * pairs(N, causal) * B * H


def bwd_flops(B, H, N, d, causal):
    return 10.0 * d * pairs(N, causal) * B * H


def decode_bytes(p):
    S, H, d = p.q.shape
    Hkv = p.kv_pool.shape[3]
    lens = p.seq_lens.tolist()
    kv = sum(lens) * Hkv * d * 2 * 2  # each valid token's K and V rows, read once
    pages = sum((L + p.page_size - 1) // p.page_size for L in lens)
    return kv + S * H * d * 2 * 2 + S * H * 4 + pages * 4 + S * 4


def src_hash(name):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(name, per_launch_units=1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    the kernel's sources are unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_sha") != src_hash(name):
        return None
    return rec.get("hbm_bytes_per_launch")


# --power SECONDS: after the timed launches, keep launching the path for that
# long while amd-smi samples board power and clocks (set by main()).
_POWER = {"seconds": 0.0, "result": None}


def power_loop(fn, seconds, idle_s=2.0):
    """Board power and graphics clocks (amd-smi) while `fn` runs back to back
    for `seconds`, after `idle_s` of the idle card.  Samples from the first
    1.5 s of the loop (clock ramp) are left out of the loaded figures."""
    import subprocess
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            t = time.time()
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=30)
                j = json.loads(r.stdout)
                g = j["gpu_data"][0] if isinstance(j, dict) else j[0]
                clk = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_")]
                samples.append((t, float(g["power"]["socket_power"]["value"]), clk))
            except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.SubprocessError):
                pass
            stop.wait(0.2)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(idle_s)
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        n += 20
    t1 = time.time()
    stop.set()
    th.join(timeout=60)
    idle = [p for t, p, c in samples if t < t0]
    load = [(p, c) for t, p, c in samples if t0 + 1.5 <= t <= t1]
    if not load:
        return {"tool": "amd-smi metric -p -c --json", "error": "no samples"}
    clocks = [sum(c) / len(c) for p, c in load if c]
    return {"tool": "amd-smi metric -p -c --json", "loop_s": round(t1 - t0, 2), "launches": n,
            "ms_per_launch_wall": round((t1 - t0) * 1e3 / n, 4),
            "idle_socket_w": round(statistics.median(idle), 1) if idle else None,
            "loaded_socket_w_mean": round(statistics.mean(p for p, c in load), 1),
            "loaded_socket_w_min": min(p for p, c in load), "loaded_socket_w_max": max(p for p, c in load),
            "loaded_gfx_mhz_mean": round(statistics.mean(clocks), 1) if clocks else None,
            "samples_loaded": len(load)}


# Untimed warm-up of each secondary record, in seconds of back-to-back calls
# (on top of its warm-up steps).  After the card has idled (inputs are built
# on the host between records), the board's power controller first lets the
# clocks overshoot and then throttles below its steady state for several
# milliseconds; a record of a short call timed inside that window measures
# the controller, not the kernel (the 4K forward: 160-180 us per launch there
# against 141 us from then on, on one card).  The headline record keeps the
# exact warm-up step count it is given; its default (DEFAULT_WARMUP launches of
# the 16K causal forward, about 0.28 s) already carries it past that window.
SECONDARY_WARM_S = 0.25
DEFAULT_STEPS, DEFAULT_WARMUP = 50, 150


def timed_launches(fn, steps, warmup, flush=None, warm_s=0.0):
    """Per-launch HIP event timings on the current stream; returns (avg_ms, median_ms, total_ms)."""
    import torch
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        for _ in range(10):
            if flush is not None:
                flush()
            fn()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record()
        fn()
        ends[i].record()
    t1.record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    if _POWER["seconds"] > 0 and _POWER["result"] is None:
        _POWER["result"] = power_loop(fn, _POWER["seconds"])
    return sum(per) / len(per), statistics.median(per), t0.elapsed_time(t1)


def bench_forward(cfg, steps, warmup, warm_s=0.0, inputs=None):
    import torch
    import exact_attention_fwd_amd as fa
    import workloads
    w = workloads.CONFIGS[cfg]
    q, k, v = inputs if inputs is not None else (t.to("cuda:0") for t in workloads.workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    fn = lambda: fa.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    avg, med, total = timed_launches(fn, steps, warmup, warm_s=warm_s)
    fl = fwd_flops(w.B, w.H, w.N, w.d, w.causal)
    del q, k, v, o, lse
    return {"workload": w.name, "kernel": fwd_kernel_name(w.d) if w.dtype == "bf16" else "fwd_f32_kernel",
            "flops_per_launch": fl, "avg_ms": avg,
            "median_ms": med, "total_ms": total, "tflops": fl / (avg * 1e-3) / 1e12,
            "frac_of_peak": fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_forward_gqa(steps, warmup, Hkv=8, warm_s=0.0):
    """The 16K causal forward with 32 query heads sharing Hkv key/value heads."""
    import torch
    import exact_attention_fwd_amd as fa
    import workloads
    w = workloads.CONFIGS["c2a"]
    q, k, v = (t.to("cuda:0") for t in workloads.gqa_inputs(w.B, w.H, Hkv, w.N, w.d, "bf16", seed=w.seed))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    fn = lambda: fa.forward(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
    avg, med, total = timed_launches(fn, steps, warmup, warm_s=warm_s)
    fl = fwd_flops(w.B, w.H, w.N, w.d, True)
    return {"workload": f"fwd_gqa_causal_1x32q{Hkv}kv_16384x128", "kernel": fwd_kernel_name(128),
            "flops_per_launch": fl, "avg_ms": avg, "median_ms": med, "tflops": fl / (avg * 1e-3) / 1e12,
            "frac_of_peak": fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_forward_rope(steps, warmup, warm_s=0.0):
    """The 16K causal forward of c2a's inputs with the rotary embedding of Q
    and K fused into the kernel (tables for positions 0..N-1, pairs (i, i+d/2)).
    Throughput counts the attention FLOPs only, as for the other forwards."""
    import torch
    import exact_attention_fwd_amd as fa
    import workloads
    w = workloads.CONFIGS["c2a"]
    q, k, v = (t.to("cuda:0") for t in workloads.workload_inputs(w))
    cos, sin = (t.to("cuda:0") for t in workloads.rope_tables(w.N, w.d))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    fn = lambda: fa.forward_rope(q, k, v, cos, sin, causal=True, scale=w.scale, out=o, lse=lse)
    avg, med, total = timed_launches(fn, steps, warmup, warm_s=warm_s)
    fl = fwd_flops(w.B, w.H, w.N, w.d, True)
    return {"workload": "fwd_rope_causal_1x32x16384x128", "kernel": fwd_kernel_name(128, rope=True),
            "flops_per_launch": fl, "avg_ms": avg, "median_ms": med, "tflops": fl / (avg * 1e-3) / 1e12,
            "frac_of_peak": fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_varlen(steps, warmup, backward=False, warm_s=0.0):
    """Packed variable-length causal forward (or backward), H=32, d=128."""
    import torch
    import exact_attention_fwd_amd as fa
    import workloads
    lens = workloads.varlen_lengths()
    H, d = 32, 128
    cu, q, k, v, do = workloads.varlen_inputs(lens, H, H, d, "bf16", seed=workloads.VARLEN_SEED, with_dout=True)
    cu, q, k, v, do = (t.to("cuda:0") for t in (cu, q, k, v, do))
    mx = max(lens)
    o, lse = fa.forward_varlen(q, k, v, cu, mx, causal=True)
    if backward:
        ws = torch.empty(int(fa.lib().fa_backward_varlen_workspace_bytes(H, q.shape[0], d)), dtype=torch.uint8,
                         device="cuda:0")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fn = lambda: fa.backward_varlen(q, k, v, o, do, lse, cu, mx, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)
        fl = sum(bwd_flops(1, H, L, d, True) for L in lens)
    else:
        fn = lambda: fa.forward_varlen(q, k, v, cu, mx, causal=True, out=o, lse=lse)
        fl = sum(fwd_flops(1, H, L, d, True) for L in lens)
    avg, med, total = timed_launches(fn, steps, warmup, warm_s=warm_s)
    return {"workload": f"{'bwd' if backward else 'fwd'}_varlen_causal_16seq_h32_d128", "seq_lens": lens,
            "total_tokens": int(sum(lens)), "flops_per_launch": fl, "avg_ms": avg, "median_ms": med,
            "tflops": fl / (avg * 1e-3) / 1e12, "frac_of_peak": fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_prefill(steps, warmup, Hkv=8, warm_s=0.0):
    """Causal chunked prefill through the paged pool, H=32 query heads, d=128."""
    import exact_attention_fwd_amd as fa
    import workloads
    chunks, ctx = workloads.prefill_shapes()
    H, d = 32, 128
    p = workloads.prefill_inputs(chunks, ctx, H=H, Hkv=Hkv, d=d, seed=workloads.PREFILL_SEED)
    q, pool, bt, sl, cu = (t.to("cuda:0") for t in (p.q, p.kv_pool, p.block_table, p.seq_lens_k,
                                                    p.cu_seqlens_q))
    o, lse = fa.prefill_paged(q, pool, bt, sl, cu, max(chunks), causal=True)
    fn = lambda: fa.prefill_paged(q, pool, bt, sl, cu, max(chunks), causal=True, out=o, lse=lse)
    avg, med, total = timed_launches(fn, steps, warmup, warm_s=warm_s)
    # visible (query, key) pairs: query i of a chunk of n over L keys sees i + L - n + 1
    vis = sum(n * (L - n) + n * (n + 1) // 2 for n, L in zip(chunks, ctx))
    fl = 4.0 * d * H * vis
    return {"workload": f"prefill_paged_causal_8x2048_h32_kv{Hkv}_d128", "chunks": chunks, "cached_keys": ctx,
            "flops_per_launch": fl, "avg_ms": avg, "median_ms": med, "tflops": fl / (avg * 1e-3) / 1e12,
            "frac_of_peak": fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_backward(steps, warmup, warm_s=0.0):
    import torch
    import exact_attention_fwd_amd as fa
    import workloads
    w = workloads.CONFIGS["c3"]
    q, k, v, do = (t.to("cuda:0") for t in workloads.workload_inputs(w))
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    ws = torch.empty(fa.backward_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda:0")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fn = lambda: fa.backward(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, workspace=ws, dq=dq, dk=dk, dv=dv)
    avg, med, total = timed_launches(fn, steps, warmup, warm_s=warm_s)
    fl = bwd_flops(w.B, w.H, w.N, w.d, w.causal)
    return {"workload": w.name, "kernels": "bwd_delta + bwd_dkdv_pipe + bwd_dq", "flops_per_call": fl, "avg_ms": avg,
            "median_ms": med, "tflops": fl / (avg * 1e-3) / 1e12,
            "frac_of_peak": fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_backward_gqa(steps, warmup, Hkv=4, warm_s=0.0):
    """The c3 causal backward ([2,16,8192,128]) with the 16 query heads sharing
    Hkv key/value heads (dK/dV summed over each group)."""
    import torch
    import exact_attention_fwd_amd as fa
    import workloads
    w = workloads.CONFIGS["c3"]
    q, k, v, do = (t.to("cuda:0") for t in workloads.gqa_inputs(w.B, w.H, Hkv, w.N, w.d, "bf16", seed=w.seed,
                                                                 with_dout=True))
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    ws = torch.empty(fa.backward_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda:0")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fn = lambda: fa.backward(q, k, v, o, do, lse, causal=True, scale=w.scale, workspace=ws, dq=dq, dk=dk, dv=dv)
    avg, med, total = timed_launches(fn, steps, warmup, warm_s=warm_s)
    fl = bwd_flops(w.B, w.H, w.N, w.d, True)
    return {"workload": f"bwd_gqa_causal_2x16q{Hkv}kv_8192x128", "kernels": "bwd_delta + bwd_dkdv_pipe + bwd_dq",
            "flops_per_call": fl, "avg_ms": avg, "median_ms": med, "tflops": fl / (avg * 1e-3) / 1e12,
            "frac_of_peak": fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_decode(steps, warmup, Hkv=None, warm_s=0.0):
    """Paged decode of the 8-sequence configuration; Hkv < 32 stores that many
    key/value heads in the pool (grouped-query decode)."""
    import torch
    import exact_attention_fwd_amd as fa
    import workloads
    w = workloads.CONFIGS["c4"]
    p = workloads.workload_inputs(w, Hkv=Hkv) if Hkv else workloads.workload_inputs(w)
    q, pool, bt, sl = (t.to("cuda:0") for t in (p.q, p.kv_pool, p.block_table, p.seq_lens))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda:0")
    ws = torch.empty(fa.decode_workspace_bytes(*q.shape, bt.shape[1]), dtype=torch.uint8, device="cuda:0")
    # Cold K/V: before every call, read 1 GiB (4x the 256 MiB last-level cache).  A read leaves the
    # caches holding clean lines; a write would leave dirty ones whose write-back lands inside the
    # timed call.
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    fn = lambda: fa.decode_paged(q, pool, bt, sl, scale=w.scale, workspace=ws, out=o, lse=lse)
    avg, med, total = timed_launches(fn, steps, warmup, flush=lambda: scratch.sum(), warm_s=warm_s)
    nbytes = decode_bytes(p)
    grouped = Hkv is not None and Hkv != w.H
    return {"workload": w.name + (f"_kv{Hkv}" if grouped else ""),
            "kernels": "decode_gqa_split + decode_merge" if grouped else "decode_split + decode_merge",
            "bytes_per_call": nbytes, "seq_lens": p.seq_lens.tolist(), "avg_ms": avg, "median_ms": med,
            "gbs": nbytes / (med * 1e-3) / 1e9, "frac_of_peak": nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "cache": "1 GiB scratch read before every call (cold K/V)"}


def bench_copy(steps, warmup, warm_s=0.0):
    """A plain 1 GiB device-to-device copy: calibrates the HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    avg, med, total = timed_launches(lambda: dst.copy_(src), steps, warmup, warm_s=warm_s)
    return {"workload": "copy_1GiB", "bytes_read": n, "bytes_written": n, "avg_ms": avg,
            "gbs": 2 * n / (avg * 1e-3) / 1e9}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(budget_s=20.0):
    """The fp64 oracle, as it stands, on whole heads of the 16K causal workload,
    with its BLAS using every core this process may run on."""
    import numpy as np  # noqa: F401
    import oracle
    import workloads
    cores = len(os.sched_getaffinity(0))
    limiter = None
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:  # pragma: no cover
        blas_threads = None
    w = workloads.CONFIGS["c2a"]
    q, k, v = workloads.workload_inputs(w)
    qf, kf, vf = (x.reshape(w.B * w.H, w.N, w.d) for x in (q, k, v))
    done, t_total = 0, 0.0
    while done < w.B * w.H:
        t0 = time.perf_counter()
        oracle.attention_forward(qf[done], kf[done], vf[done], causal=True, scale=w.scale)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    if limiter is not None:
        limiter.restore_original_limits()
    fl = fwd_flops(1, 1, w.N, w.d, True) * done
    return {"value": fl / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "blas_threads": blas_threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} heads of {w.name} (full causal forward per head, fp64 numpy), "
                      f"{t_total:.1f} s; value = algorithmic flops of the sample / wall time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    ap.add_argument("--only", choices=["fwd", "fwd32k", "fwdnc", "fwd4k", "bwd", "decode", "copy", "fwdgqa",
                                       "fwdvarlen", "bwdvarlen", "decodegqa", "prefill", "bwdgqa", "fwdrope"], default=None,
                    help="run one path only (for profiler runs); prints its record")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-s", type=float, default=None, metavar="SECONDS",
                    help="with --only: untimed seconds of back-to-back calls after the warm-up steps "
                         f"(default: 0 for fwd, as the headline record; {SECONDARY_WARM_S} for the others, as their records)")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="with --only: afterwards launch the path back to back for SECONDS while amd-smi "
                         "samples board power and clocks (decode: without the cache flush)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.only:
        _POWER["seconds"] = args.power
        ws = args.warm_s if args.warm_s is not None else (0.0 if args.only == "fwd" else SECONDARY_WARM_S)
        rec = {"fwd": lambda: bench_forward("c2a", args.steps, args.warmup, warm_s=ws),
               "fwd32k": lambda: bench_forward("c2b", args.steps, args.warmup, warm_s=ws),
               "fwdnc": lambda: bench_forward("c2c", args.steps, args.warmup, warm_s=ws),
               "fwd4k": lambda: bench_forward("c1", args.steps, args.warmup, warm_s=ws),
               "bwd": lambda: bench_backward(args.steps, args.warmup, warm_s=ws),
               "copy": lambda: bench_copy(args.steps, args.warmup, warm_s=ws),
               "decode": lambda: bench_decode(args.steps, args.warmup, warm_s=ws),
               "fwdgqa": lambda: bench_forward_gqa(args.steps, args.warmup, warm_s=ws),
               "fwdvarlen": lambda: bench_varlen(args.steps, args.warmup, warm_s=ws),
               "bwdvarlen": lambda: bench_varlen(args.steps, args.warmup, backward=True, warm_s=ws),
               "decodegqa": lambda: bench_decode(args.steps, args.warmup, Hkv=8, warm_s=ws),
               "prefill": lambda: bench_prefill(args.steps, args.warmup, warm_s=ws),
               "bwdgqa": lambda: bench_backward_gqa(args.steps, args.warmup, warm_s=ws),
               "fwdrope": lambda: bench_forward_rope(args.steps, args.warmup, warm_s=ws)}[args.only]()
        rec["warm_s"] = ws
        if _POWER["result"] is not None:
            rec["power"] = _POWER["result"]
        print(json.dumps(rec), flush=True)
        return

    print("# forward c2a (headline)", file=sys.stderr, flush=True)
    main_rec = bench_forward("c2a", args.steps, args.warmup)
    secondary = []
    ws = SECONDARY_WARM_S
    for name, f in (("fwd c1", lambda: bench_forward("c1", args.steps, args.warmup, warm_s=ws)),
                    ("fwd c2b", lambda: bench_forward("c2b", max(5, args.steps // 2), 2, warm_s=ws)),
                    ("fwd c2c", lambda: bench_forward("c2c", max(5, args.steps // 2), 2, warm_s=ws)),
                    ("bwd c3", lambda: bench_backward(max(5, args.steps // 2), 2, warm_s=ws)),
                    ("decode c4", lambda: bench_decode(args.steps, args.warmup, warm_s=ws)),
                    ("fwd gqa 32q/8kv", lambda: bench_forward_gqa(max(5, args.steps // 2), 2, warm_s=ws)),
                    ("bwd gqa 16q/4kv", lambda: bench_backward_gqa(max(5, args.steps // 2), 2, warm_s=ws)),
                    ("fwd varlen", lambda: bench_varlen(max(5, args.steps // 2), 2, warm_s=ws)),
                    ("bwd varlen", lambda: bench_varlen(max(5, args.steps // 2), 2, backward=True, warm_s=ws)),
                    ("decode c4 gqa 32q/8kv", lambda: bench_decode(args.steps, args.warmup, Hkv=8, warm_s=ws)),
                    ("prefill paged", lambda: bench_prefill(max(5, args.steps // 2), 2, warm_s=ws)),
                    ("fwd rope", lambda: bench_forward_rope(max(5, args.steps // 2), 2, warm_s=ws))):
        print(f"# {name}", file=sys.stderr, flush=True)
        secondary.append(dict(f(), warm_s=ws))
        torch.cuda.empty_cache()
    base = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        base = cpu_baseline()

    fl = main_rec["flops_per_launch"]
    achieved = fl / (main_rec["avg_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(main_rec["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_rec["total_ms"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16",
        "config": {"workload": main_rec["workload"], "B": 1, "H": 32, "N": 16384, "d": 128, "causal": True,
                   "scale": 1 / math.sqrt(128)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic_for(main_rec["kernel"]),
                     "kernel": main_rec["kernel"], "avg_launch_ms": round(main_rec["avg_ms"], 4)},
        "cpu_baseline": base,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
