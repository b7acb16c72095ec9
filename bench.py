"""Benchmark of the MXFP8 hot path on one MI355X.

Default step (the Qwen3-8B qkv_proj layer, 4096 tokens): quantize W[6144x4096]
and X[4096x4096] along K, repack W into the GEMM layout, and run the MXFP8
GEMM Y = X W^T with bf16 output.  Inputs are resident in HBM before the timed
region; R input/output sets are rotated so the working set (> 512 MB) does not
sit in the 256 MB Infinity Cache.  In the timed steps the GEMM launch is
bracketed by HIP events on the stream it runs on, so its average duration is
measured live; the quantize and repack kernels are timed the same way in a
pass of their own after the timed region (an event record costs GPU time
between kernels).  `value` is the whole step's throughput (2MNK / step time).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload qkv|mlp|moe|moe_train|sync|sweep]
                    [--no-cpu-baseline]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MXFP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 / MXFP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0
Q_BYTES_PER_ELT = 2 + 1 + 1 / 32     # quantize: BF16 in, E4M3 + E8M0 out
REPACK_BYTES_PER_ELT = 2 * (1 + 1 / 32)

def measured_gemm_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (scaled by the copy-kernel factors), if it was taken on
    the GEMM source that is built now; None otherwise."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "qkv_step_hbm_traffic.md")
    src = os.path.join(ROOT, "mxfp8_block_scaled_05_amd", "csrc", "gemm.hip")
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines() if ": " in line
                      and line.split(": ", 1)[0] in ("traffic_bytes_per_launch", "gemm_source_sha256"))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if fields.get("gemm_source_sha256", "").strip() != sha:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _bf16_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def settle(step, seconds):
    """Run `step()` (untimed) until `seconds` of wall time have passed: the
    GPU's clocks ramp for tens of milliseconds after it leaves idle (measured:
    the qkv GEMM takes ~114 us on average over its first 50 launches and
    ~102 us once settled), so the warm-up ends in steady state whatever W is.
    Returns the seconds spent."""
    import torch
    if seconds <= 0:
        return 0.0
    t0 = time.perf_counter()
    n = 0
    while True:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return time.perf_counter() - t0


class KernelTimer:
    """HIP events around each launch, on the current stream."""

    def __init__(self):
        self.pending = {}

    def time(self, name, fn):
        import torch
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.pending.setdefault(name, []).append((s, e))
        return out

    def averages_us(self):
        return {k: 1e3 * float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in self.pending.items()}

    def medians_us(self):
        return {k: 1e3 * float(np.median([s.elapsed_time(e) for s, e in v])) for k, v in self.pending.items()}

    def reset(self):
        self.pending = {}


def host_description():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "omp_num_threads": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))}


def copy_reference_us(dev, nbytes: int, reps: int = 30) -> float:
    """Median time of a plain device copy moving `nbytes` (half read, half
    written), rotated over buffers so that it reads from HBM like the timed
    kernels: the HBM rate reachable at that transfer size."""
    import torch
    half = nbytes // 2 // 4096 * 4096
    R = max(3, int(700e6 // nbytes) + 1)
    srcs = [torch.ones(half, dtype=torch.uint8, device=dev) for _ in range(R)]
    dsts = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(R)]
    for i in range(R):
        dsts[i].copy_(srcs[i])
    torch.cuda.synchronize()
    ev = []
    for it in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dsts[it % R].copy_(srcs[it % R])
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))


def bench_qkv(args, dev):
    import torch
    import mxfp8_block_scaled_05_amd as mx
    import workloads as wl

    M, K = 4096, wl.QWEN3_8B["hidden"]
    N = wl.QWEN3_8B["qkv"]
    d = wl.qkv(0, tokens=M)
    per_set = (N * K + M * K) * 2 + (N * K + M * K) + N * K + M * K + M * N * 2
    # 8 sets (1.6 GB): each op's inputs over the sets exceed the 256 MB
    # Infinity Cache, so back-to-back launches of one op over the sets read HBM
    R = max(8, int(np.ceil(600e6 / per_set)))
    sets = []
    for r in range(R):
        # distinct bytes per set: rotate the seeded tensors
        X = _bf16_dev(np.roll(d["X"], r, axis=0), dev)
        W = _bf16_dev(np.roll(d["W"], r, axis=0), dev)
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        xs = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
        w = mx.PackedWeight(torch.empty(mx.packed_bytes(1, N, K, 0), dtype=torch.uint8, device=dev),
                            torch.empty(mx.packed_bytes(1, N, K, 1), dtype=torch.uint8, device=dev),
                            1, N, K)
        # X quantized straight into the GEMM's packed operand layout
        a = mx.PackedWeight(torch.empty(mx.packed_bytes(1, M, K, 0), dtype=torch.uint8, device=dev),
                            torch.empty(mx.packed_bytes(1, M, K, 1), dtype=torch.uint8, device=dev),
                            1, M, K)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        sets.append((X, W, xq, xs, wq, ws, w, a, y))
    torch.cuda.synchronize()
    timer = KernelTimer()

    def step(i, timed):
        # timed: HIP events around the listed ops.  Each event record costs
        # ~3 us of GPU time between the kernels (measured: the step takes
        # 161 us with events around all four ops, 139-144 us with events
        # around the GEMM only, 133 us with none), so the timed steps bracket
        # only the GEMM, whose live duration the roofline needs; the HBM-bound
        # kernels are timed in a pass of their own after the timed region.
        X, W, xq, xs, wq, ws, w, a, y = sets[i % R]
        t = timer.time if "all" in timed else (lambda name, fn: fn())
        # W along K into its canonical grid and X along K straight into the
        # GEMM's packed operand layout, one launch (mxfp8_quantize_many_layouts)
        t("quantize_WX", lambda: mx.quantize_many_layouts_([(W, (wq, ws)), (X, a)]))
        t("repack_W", lambda: mx.repack_(wq, ws, w))
        if timed:
            timer.time("gemm", lambda: mx.gemm_packed(a, w, torch.bfloat16, out=y))
        else:
            mx.gemm_packed(a, w, torch.bfloat16, out=y)

    # the settle phase rotates the input sets like the timed steps, so every
    # launch a kernel trace of this command averages reads from HBM
    rot = [0]

    def settle_step():
        step(rot[0], ())
        rot[0] += 1
    settled = settle(settle_step, args.settle_s)
    gc.disable()   # no collector pauses between the timing events
    for i in range(args.warmup):
        step(i, ("gemm",))
    torch.cuda.synchronize()
    timer.reset()
    # timed region: K steps, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ("gemm",))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = timer.averages_us()
    med = timer.medians_us()
    # per-kernel pass (outside the timed region): events around every op
    timer.reset()
    for i in range(min(args.steps, 100)):
        step(i, ("all",))
    torch.cuda.synchronize()
    gc.enable()
    avg_all = timer.averages_us()
    med_all = timer.medians_us()
    # HBM-bound ops: each timed as a batch of back-to-back launches over the
    # rotated sets between two events (an event pair around one short launch
    # adds a few microseconds of its own); per-launch time = batch / count
    batch = {}
    B = 4 * R

    def qw(s):
        mx.quantize_into(s[1], 1, s[4], s[5])

    def qwx(s):
        mx.quantize_many_layouts_([(s[1], (s[4], s[5])), (s[0], s[7])])

    def rp(s):
        mx.repack_(s[4], s[5], s[6])
    for k, fns in (("quantize_W", (qw,)), ("quantize_X", (lambda s: mx.quantize_into(s[0], 1, s[2], s[3]),)),
                   ("quantize_WX", (qwx,)), ("repack_W_cold", (rp,)), ("quantize_WX+repack_W", (qwx, rp))):
        for fn in fns:
            fn(sets[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(B):
            for fn in fns:
                fn(sets[i % R])
        e1.record()
        torch.cuda.synchronize()
        batch[k] = 1e3 * e0.elapsed_time(e1) / B
    # in the step, repack reads the grid quantize_W has just written: its
    # share of a quantize + repack pair
    batch["repack_W"] = batch["quantize_WX+repack_W"] - batch["quantize_WX"]
    for k in ("quantize_WX", "repack_W"):
        avg[k], med[k] = batch[k], med_all[k]
    for k in ("quantize_W", "quantize_X"):
        avg[k] = batch[k]
    # the accurate GEMM (mxfp8_gemm_accurate: BF16 matrix instructions on
    # exactly converted operands) on the same rotated inputs, its own pass
    timer.reset()
    for i in range(R):          # canonical X grids for the reference GEMM passes
        X, W, xq, xs, wq, ws, w, a, y = sets[i]
        mx.quantize_into(X, 1, xq, xs)
    for i in range(min(args.steps, 20)):
        X, W, xq, xs, wq, ws, w, a, y = sets[i % R]
        timer.time("gemm_accurate", lambda: mx.gemm(xq, xs, w, torch.bfloat16, out=y, accurate=True))
    # the step as it would be with X's canonical grid (mxfp8_quantize_many,
    # mxfp8_gemm): events around the GEMM only, its inputs as fresh as above
    for i in range(max(args.steps, 20)):
        X, W, xq, xs, wq, ws, w, a, y = sets[i % R]
        mx.quantize_many_([(W, wq, ws), (X, xq, xs)])
        mx.repack_(wq, ws, w)
        timer.time("gemm_canonical_A", lambda: mx.gemm(xq, xs, w, torch.bfloat16, out=y))
    torch.cuda.synchronize()
    acc_us = timer.averages_us()["gemm_accurate"]
    can_us = timer.averages_us()["gemm_canonical_A"]
    ms_per_step = 1e3 * wall / args.steps
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (avg["gemm"] * 1e-6) / 1e12
    kern = {
        "quantize_WX": _bw(avg["quantize_WX"], (N + M) * K * Q_BYTES_PER_ELT),
        "quantize_W": _bw(avg["quantize_W"], N * K * Q_BYTES_PER_ELT),
        "quantize_X": _bw(avg["quantize_X"], M * K * Q_BYTES_PER_ELT),
        "repack_W": _bw(avg["repack_W"], N * K * REPACK_BYTES_PER_ELT),
        "gemm": {"us": round(avg["gemm"], 2), "TFLOP/s": round(gemm_tflops, 1),
                 "frac_mxfp8_peak": round(gemm_tflops / MXFP8_PEAK_TFLOPS, 4),
                 "us_with_events_around_every_op": round(avg_all["gemm"], 2)},
    }
    kern["gemm_accurate"] = _gemm_rate(acc_us, M, N, K)
    kern["gemm_canonical_A"] = _gemm_rate(can_us, M, N, K)
    kern["gemm_canonical_A"]["note"] = ("mxfp8_gemm on X's canonical grid (its copies gather 8 rows per "
                                        "instruction) in the same step with mxfp8_quantize_many, for reference")
    kern["gemm"]["median_us"] = round(med["gemm"], 2)
    for k in ("quantize_WX", "repack_W"):
        kern[k]["us_events_around_each_launch"] = round(avg_all[k], 2)
    kern["quantize_W"]["note"] = kern["quantize_X"]["note"] = \
        "one tensor per launch into its canonical grid (mxfp8_quantize), for reference; the step quantizes both in one launch"
    kern["repack_W"]["us_cold_input"] = round(batch["repack_W_cold"], 2)
    # context for the HBM-bound kernels: a plain copy of the same bytes, cold
    for k, nbytes in (("quantize_WX", (N + M) * K * Q_BYTES_PER_ELT), ("quantize_W", N * K * Q_BYTES_PER_ELT),
                      ("quantize_X", M * K * Q_BYTES_PER_ELT), ("repack_W", N * K * REPACK_BYTES_PER_ELT)):
        kern[k]["same_bytes_copy_us"] = round(copy_reference_us(dev, int(nbytes)), 2)
    out = {
        "metric": "MXFP8 GEMM TFLOP/s (% MX peak) + quantize GB/s (% HBM) at Qwen3-8B shapes",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": round(settled, 3),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3/e8m0, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded N(0,1) activations with 1% x20 outliers, N(0,0.02) weights)",
        "config": {"workload": "qwen3-8b qkv_proj: quantize W[6144x4096] (canonical grid) + X[4096x4096] (the "
                               "GEMM's packed operand layout) along K in one mxfp8_quantize_many_layouts launch, "
                               "repack W, MXFP8 GEMM (mxfp8_gemm_packed) -> bf16",
                   "M": M, "N": N, "K": K, "rotated_sets": R},
        "kernels": kern,
        "kernels_note": "gemm: HIP events around every GEMM launch of the timed steps; quantize and "
                        "repack: a batch of %d back-to-back launches over the %d rotated sets between two "
                        "events, per launch (repack_W: a batch of quantize_WX + repack_W pairs less the "
                        "quantize_WX batch, since in the step repack reads the grid just written; "
                        "us_events_around_each_launch: events around every op of min(steps, 100) steps); "
                        "gemm_accurate, gemm_canonical_A: passes of their own" % (4 * R, R),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": MXFP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / MXFP8_PEAK_TFLOPS, 4),
                     "traffic": measured_gemm_traffic()},
    }
    return out


def run_timed(ops, args, live=()):
    """Run `ops` (a list of (name, fn)) as one step: W warmup steps, then K
    timed steps bracketed by synchronizations, with HIP events only around
    the ops named in `live` (an event record costs GPU time between kernels);
    then a pass of min(K, 50) steps with events around every op.  Returns (ms
    per step from the host clock over the timed steps, {name: avg us}), the
    averages of `live` ops from the timed steps, the others from that pass."""
    import torch
    timer = KernelTimer()

    def plain():
        for _, fn in ops:
            fn()

    def one(names):
        for name, fn in ops:
            if name in names:
                timer.time(name, fn)
            else:
                fn()
    settle(plain, getattr(args, "settle_s", 0.0))
    gc.disable()
    for _ in range(args.warmup):
        one(live)
    torch.cuda.synchronize()
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one(live)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_live = timer.averages_us()
    timer.reset()
    every = {name for name, _ in ops}
    for _ in range(min(args.steps, 50)):
        one(every)
    torch.cuda.synchronize()
    gc.enable()
    avg = timer.averages_us()
    avg.update(avg_live)
    return 1e3 * wall / args.steps, avg


def _line(metric, value, unit, args, ms, dtype, config, **extra):
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic (seeded; recipe in workloads/)", "config": config}
    out.update(extra)
    return out


def _gemm_rate(us, M, N, K):
    tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
    return {"us": round(us, 2), "TFLOP/s": round(tf, 1), "frac_mxfp8_peak": round(tf / MXFP8_PEAK_TFLOPS, 4)}


def bench_mlp(args, dev):
    """Qwen3-8B MLP learner micro-batch (8192 tokens): per step, quantize each
    of the two weights and the four activation/gradient tensors once, along
    both axes, straight into the GEMM's packed operand layouts (blocked along
    the reduction axis of each product that reads it), then run the six GEMMs
    (fprop, dgrad, wgrad for gate_up and down) on packed operands.
    fprop/dgrad -> bf16, wgrad -> fp32.  The working set (> 2.5 GB) is far
    larger than the Infinity Cache.  The unfused composition (each tensor
    quantized per axis into its canonical grid, the weights repacked, the
    GEMMs reading A from the canonical grid) is timed in a pass of its own."""
    import torch
    import mxfp8_block_scaled_05_amd as mx
    import workloads as wl

    T = 8192
    d = wl.mlp(0, tokens=T)
    H, I2 = d["W_gu"].shape[1], d["W_gu"].shape[0]
    I = d["W_d"].shape[1]
    t = {k: _bf16_dev(v, dev) for k, v in d.items()}
    del d

    def qbuf(rows, cols, axis):
        r, c = (rows, cols) if axis == 1 else (cols, rows)
        return (torch.empty((r, c), dtype=torch.uint8, device=dev),
                torch.empty((r, c // 32), dtype=torch.uint8, device=dev))

    def pbuf(n, k):
        return mx.PackedWeight(torch.empty(mx.packed_bytes(1, n, k, 0), dtype=torch.uint8, device=dev),
                               torch.empty(mx.packed_bytes(1, n, k, 1), dtype=torch.uint8, device=dev),
                               1, n, k)

    names = ("W_gu", "W_d", "X", "h", "dY_gu", "dY_d")
    # P[name, 1]: the tensor's rows as GEMM rows, blocked along its columns;
    # P[name, 0]: its columns as GEMM rows, blocked along its rows
    P = {}
    for name in names:
        r, c = t[name].shape
        P[name, 1], P[name, 0] = pbuf(r, c), pbuf(c, r)
    out = {"fprop_gu": torch.empty((T, I2), dtype=torch.bfloat16, device=dev),
           "fprop_d": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
           "dgrad_d": torch.empty((T, I), dtype=torch.bfloat16, device=dev),
           "dgrad_gu": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
           "wgrad_d": torch.empty((H, I), dtype=torch.float32, device=dev),
           "wgrad_gu": torch.empty((I2, H), dtype=torch.float32, device=dev)}
    gemms = {  # name: (A, B) as (tensor, axis) of P, M, N, K, out dtype
        "fprop_gu": (("X", 1), ("W_gu", 1), T, I2, H, torch.bfloat16),
        "fprop_d": (("h", 1), ("W_d", 1), T, H, I, torch.bfloat16),
        "dgrad_d": (("dY_d", 1), ("W_d", 0), T, I, H, torch.bfloat16),
        "dgrad_gu": (("dY_gu", 1), ("W_gu", 0), T, H, I2, torch.bfloat16),
        "wgrad_d": (("dY_d", 0), ("h", 0), H, I, T, torch.float32),
        "wgrad_gu": (("dY_gu", 0), ("X", 0), I2, H, T, torch.float32),
    }
    # the step: six dual quantizes (one read each), six packed GEMMs
    ops = []
    q_bytes = {}
    for name in names:
        key = "quantize_dual_packed_" + name
        ops.append((key, lambda x=t[name], a=P[name, 1], b=P[name, 0]: mx.quantize_dual_packed_(x, a, b)))
        q_bytes[key] = t[name].numel() * (2 + 2 * (1 + 1 / 32))
    for key, (A, B, M, N, K, dt) in gemms.items():
        ops.append(("gemm_" + key, lambda A=P[A], B=P[B], dt=dt, o=out[key]: mx.gemm_packed(A, B, dt, out=o)))
    # unfused composition: every tensor quantized per axis into its canonical
    # grid, the weights repacked, the GEMMs reading A from the canonical grid
    Q = {(name, ax): qbuf(*t[name].shape, ax) for name in names for ax in (1, 0)}
    unfused = []
    for (name, ax), (q, sc) in Q.items():
        key = "quantize_%s_axis%d" % (name, ax)
        unfused.append((key, lambda x=t[name], a=ax, q=q, sc=sc: mx.quantize_into(x, a, q, sc)))
    for name in ("W_gu", "W_d"):
        for ax in (1, 0):
            unfused.append(("repack_%s_axis%d" % (name, ax),
                            lambda q=Q[name, ax][0], sc=Q[name, ax][1], w=P[name, ax]: mx.repack_(q, sc, w)))
    for key, (A, B, M, N, K, dt) in gemms.items():
        # weights from their repacked layout, wgrad's B from its canonical grid
        Bw = P[B] if B[0].startswith("W_") else Q[B]
        unfused.append(("gemm_%s_canonical_A" % key,
                        lambda A=Q[A], B=Bw, dt=dt, o=out[key]: mx.gemm(A[0], A[1], B, dt, out=o)))
    torch.cuda.synchronize()
    ms, avg = run_timed(ops, args, live=("gemm_fprop_gu",))
    _, avg_unf = run_timed(unfused, argparse.Namespace(steps=max(2, args.steps // 2), warmup=1))
    # the whole micro-batch (12 launches) captured once and replayed
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _, fn in ops:
            fn()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(max(2, args.steps // 2)):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / max(2, args.steps // 2)
    del graph
    flops = sum(2.0 * M * N * K for (_, _, M, N, K, _) in gemms.values())
    kern = {}
    for key, nbytes in q_bytes.items():
        kern[key] = _bw(avg[key], nbytes)
    # the largest tensor quantized along each axis on its own (unfused pass)
    for ax in (1, 0):
        key = "quantize_dY_gu_axis%d" % ax
        kern[key + "_unfused"] = _bw(avg_unf[key], t["dY_gu"].numel() * Q_BYTES_PER_ELT)
    for key, (_, _, M, N, K, _) in gemms.items():
        kern["gemm_" + key] = _gemm_rate(avg["gemm_" + key], M, N, K)
    canon = {key: _gemm_rate(avg_unf["gemm_%s_canonical_A" % key], M, N, K)
             for key, (_, _, M, N, K, _) in gemms.items()}
    gemm_us = sum(avg["gemm_" + k] for k in gemms)
    canon_us = sum(avg_unf["gemm_%s_canonical_A" % k] for k in gemms)
    quant_us = sum(avg[k] for k in avg if not k.startswith("gemm_"))
    unfused_us = sum(v for k, v in avg_unf.items() if not k.startswith("gemm_"))
    top = kern["gemm_fprop_gu"]
    return _line("MXFP8 GEMM TFLOP/s (% MX peak) + quantize GB/s (% HBM) at Qwen3-8B shapes",
                 round(flops / (ms * 1e-3) / 1e12, 2), "TFLOP/s", args, ms,
                 "mxfp8-e4m3/e8m0, fp32 accumulate, bf16 out (fprop/dgrad), fp32 out (wgrad)",
                 {"workload": "qwen3-8b MLP learner micro-batch, 8192 tokens: weights, activations and "
                              "gradients quantized along both axes (one read each) straight into the "
                              "packed operand layouts, 6 GEMMs on packed operands",
                  "tokens": T, "hidden": H, "inter": I},
                 kernels=kern,
                 summary={"gemm_us": round(gemm_us, 1),
                          "gemm_TFLOP/s": round(flops / (gemm_us * 1e-6) / 1e12, 1),
                          "graph_replay_ms_per_step": round(graph_ms, 4),
                          "quantize_and_layout_us": round(quant_us, 1),
                          "unfused_quantize_and_layout_us": round(unfused_us, 1),
                          "canonical_A_gemm_us": round(canon_us, 1),
                          "canonical_A_gemms": canon},
                 roofline={"bound": "mfma", "achieved": top["TFLOP/s"], "peak": MXFP8_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": top["frac_mxfp8_peak"], "traffic": None,
                           "kernel": "gemm fprop gate_up 8192x24576x4096"})


def bench_moe(args, dev):
    """Qwen3-30B-A3B MoE layer forward (8192 tokens, 128 experts, Zipf(1.1)
    top-8, groups padded to 32): quantize the gathered gate_up input straight
    into the GEMM's packed operand layout, grouped GEMM gate_up -> bf16
    (mxfp8_grouped_gemm_packed), the same for the down input and GEMM.
    Expert weights are quantized and repacked beforehand (weight sync, timed
    separately); offsets stay on the device.  The canonical-A grouped GEMMs
    over the same inputs are timed in a pass of their own, for reference."""
    import torch
    import mxfp8_block_scaled_05_amd as mx
    import workloads as wl

    d = wl.moe(0)
    G, I2, H = d["W_gu"].shape
    I = d["W_d"].shape[2]
    Mt = int(d["offsets"][-1])
    real = int(d["counts"].sum())
    W_gu = _bf16_dev(d["W_gu"].reshape(G * I2, H), dev)
    W_d = _bf16_dev(d["W_d"].reshape(G * H, I), dev)
    A_gu = _bf16_dev(d["A_gu"], dev)
    A_d = _bf16_dev(d["A_d"], dev)
    offs = torch.from_numpy(d["offsets"]).to(dev)
    del d
    wgu_q = torch.empty((G * I2, H), dtype=torch.uint8, device=dev)
    wgu_s = torch.empty((G * I2, H // 32), dtype=torch.uint8, device=dev)
    wd_q = torch.empty((G * H, I), dtype=torch.uint8, device=dev)
    wd_s = torch.empty((G * H, I // 32), dtype=torch.uint8, device=dev)
    P_gu = mx.PackedWeight(torch.empty(mx.packed_bytes(G, I2, H, 0), dtype=torch.uint8, device=dev),
                           torch.empty(mx.packed_bytes(G, I2, H, 1), dtype=torch.uint8, device=dev), G, I2, H)
    P_d = mx.PackedWeight(torch.empty(mx.packed_bytes(G, H, I, 0), dtype=torch.uint8, device=dev),
                          torch.empty(mx.packed_bytes(G, H, I, 1), dtype=torch.uint8, device=dev), G, H, I)
    agu_q = torch.empty((Mt, H), dtype=torch.uint8, device=dev)
    agu_s = torch.empty((Mt, H // 32), dtype=torch.uint8, device=dev)
    ad_q = torch.empty((Mt, I), dtype=torch.uint8, device=dev)
    ad_s = torch.empty((Mt, I // 32), dtype=torch.uint8, device=dev)
    agu_p = mx.PackedWeight(torch.empty(mx.packed_bytes(1, Mt, H, 0), dtype=torch.uint8, device=dev),
                            torch.empty(mx.packed_bytes(1, Mt, H, 1), dtype=torch.uint8, device=dev), 1, Mt, H)
    ad_p = mx.PackedWeight(torch.empty(mx.packed_bytes(1, Mt, I, 0), dtype=torch.uint8, device=dev),
                           torch.empty(mx.packed_bytes(1, Mt, I, 1), dtype=torch.uint8, device=dev), 1, Mt, I)
    y_gu = torch.empty((Mt, I2), dtype=torch.bfloat16, device=dev)
    y_d = torch.empty((Mt, H), dtype=torch.bfloat16, device=dev)
    sync_ops = [
        ("sync_quantize_W_gu", lambda: mx.quantize_into(W_gu, 1, wgu_q, wgu_s)),
        ("sync_repack_W_gu", lambda: mx.repack_(wgu_q.view(G, I2, H), wgu_s.view(G, I2, H // 32), P_gu)),
        ("sync_quantize_W_d", lambda: mx.quantize_into(W_d, 1, wd_q, wd_s)),
        ("sync_repack_W_d", lambda: mx.repack_(wd_q.view(G, H, I), wd_s.view(G, H, I // 32), P_d)),
    ]
    ops = [
        ("quantize_A_gu", lambda: mx.quantize_many_layouts_([(A_gu, agu_p)])),
        ("grouped_gemm_gate_up", lambda: mx.grouped_gemm_packed(agu_p, P_gu, offs, torch.bfloat16, out=y_gu)),
        ("quantize_A_d", lambda: mx.quantize_many_layouts_([(A_d, ad_p)])),
        ("grouped_gemm_down", lambda: mx.grouped_gemm_packed(ad_p, P_d, offs, torch.bfloat16, out=y_d)),
    ]
    ref_ops = [
        ("quantize_A_gu_canonical", lambda: mx.quantize_into(A_gu, 1, agu_q, agu_s)),
        ("grouped_gemm_gate_up_canonical_A", lambda: mx.grouped_gemm(agu_q, agu_s, P_gu, offs, torch.bfloat16,
                                                                     out=y_gu)),
        ("quantize_A_d_canonical", lambda: mx.quantize_into(A_d, 1, ad_q, ad_s)),
        ("grouped_gemm_down_canonical_A", lambda: mx.grouped_gemm(ad_q, ad_s, P_d, offs, torch.bfloat16, out=y_d)),
    ]
    torch.cuda.synchronize()
    sync_ms, sync_avg = run_timed(sync_ops, argparse.Namespace(steps=max(3, args.steps // 10), warmup=1))
    ms, avg = run_timed(ops, args, live=("grouped_gemm_gate_up",))
    _, ref_avg = run_timed(ref_ops, argparse.Namespace(steps=max(3, args.steps // 2), warmup=1))
    flops_gu = 2.0 * real * I2 * H
    flops_d = 2.0 * real * H * I
    eb = 1 + 1 / 32
    bytes_gu = G * I2 * H * eb + Mt * H * eb + Mt * I2 * 2
    bytes_d = G * H * I * eb + Mt * I * eb + Mt * H * 2
    kern = {"quantize_A_gu": _bw(avg["quantize_A_gu"], Mt * H * Q_BYTES_PER_ELT),
            "quantize_A_d": _bw(avg["quantize_A_d"], Mt * I * Q_BYTES_PER_ELT)}
    for key, fl, by in (("grouped_gemm_gate_up", flops_gu, bytes_gu), ("grouped_gemm_down", flops_d, bytes_d)):
        us = avg[key]
        tf = fl / (us * 1e-6) / 1e12
        gbs = by / (us * 1e-6) / 1e9
        kern[key] = {"us": round(us, 2), "TFLOP/s": round(tf, 1), "frac_mxfp8_peak": round(tf / MXFP8_PEAK_TFLOPS, 4),
                     "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "roofline_us": round(max(fl / MXFP8_PEAK_TFLOPS / 1e12, by / HBM_PEAK_GBS / 1e9) * 1e6, 1)}
    for key, fl in (("grouped_gemm_gate_up_canonical_A", flops_gu), ("grouped_gemm_down_canonical_A", flops_d)):
        tf = fl / (ref_avg[key] * 1e-6) / 1e12
        kern[key] = {"us": round(ref_avg[key], 2), "TFLOP/s": round(tf, 1),
                     "frac_mxfp8_peak": round(tf / MXFP8_PEAK_TFLOPS, 4),
                     "note": "mxfp8_grouped_gemm over the canonical grid of the same rows, a pass of its own"}
    for key in ("sync_quantize_W_gu", "sync_quantize_W_d"):
        n = G * I2 * H if key.endswith("gu") else G * H * I
        kern[key] = _bw(sync_avg[key], n * Q_BYTES_PER_ELT)
    for key in ("sync_repack_W_gu", "sync_repack_W_d"):
        n = G * I2 * H if key.endswith("gu") else G * H * I
        kern[key] = _bw(sync_avg[key], n * REPACK_BYTES_PER_ELT)
    top = kern["grouped_gemm_gate_up"]
    return _line("MXFP8 GEMM TFLOP/s (% MX peak) + quantize GB/s (% HBM) at Qwen3-8B shapes",
                 round((flops_gu + flops_d) / (ms * 1e-3) / 1e12, 2), "TFLOP/s", args, ms,
                 "mxfp8-e4m3/e8m0, fp32 accumulate, bf16 out",
                 {"workload": "qwen3-30b-a3b MoE layer forward, 8192 tokens, 128 experts, Zipf(1.1) top-8, "
                              "groups padded to 32: quantize (into the packed operand layout) + grouped GEMM "
                              "gate_up, the same for down",
                  "tokens": 8192, "experts": G, "rows_real": real, "rows_padded": Mt},
                 kernels=kern, flops_basis="unpadded rows (padded FLOPs are %.1f%% more)" % (100.0 * (Mt / real - 1)),
                 roofline={"bound": "mfma", "achieved": top["TFLOP/s"], "peak": MXFP8_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": top["frac_mxfp8_peak"], "traffic": None,
                           "kernel": "grouped gemm gate_up", "hbm_frac": top["frac_hbm_peak"]})


def bench_moe_train(args, dev):
    """Qwen3-30B-A3B MoE expert layer, one learner micro-batch of 8192 tokens
    (128 experts, Zipf(1.1) top-8, groups padded to 32): forward, data
    gradients and weight gradients of gate_up and down, all in MXFP8.
      weights (per step): gate_up and down quantized from one read each along
        K into the packed layout and along N per expert straight into the
        packed layout of the transposed weights (for dgrad);
      forward: X gathered by routing + quantized in one pass (the fused
        permute) straight into the packed operand layout, grouped gate_up;
        h quantized along both axes, grouped down;
      backward: dY quantized along both axes -> dgrad down (grouped GEMM vs
        W_d^T), wgrad down (grouped-K GEMM dY^T h); dH quantized along both
        axes -> dgrad gate_up, wgrad gate_up (grouped-K GEMM dH^T X).
    The forward and data-gradient GEMMs read A in the packed layout
    (mxfp8_grouped_gemm_packed); the token-blocked (axis-0) grids that feed
    the weight gradients are written regrouped, every expert's tokens
    starting on a multiple of 128 (mxfp8_quantize_dual_grouped_packed), so
    the weight-gradient GEMMs run aligned.  Timed beside the step: the
    weight-gradient GEMMs over the 32-padded grids and over the regrouped
    grids in the packed layout (mxfp8_grouped_gemm_wgrad_packed), and the
    other four with A from the canonical grids.
    The activation function between gate_up and down is outside the MXFP8
    path; h and dH are drawn as N(0,1) and N(0,1)*2^-10 on real rows."""
    import torch
    import mxfp8_block_scaled_05_amd as mx
    import workloads as wl

    d = wl.moe(0)
    G, I2, H = d["W_gu"].shape
    I = d["W_d"].shape[2]
    offs_np = d["offsets"]
    Mt = int(offs_np[-1])
    real = int(d["counts"].sum())
    rng = np.random.default_rng(1)
    realrows = d["row_token"] >= 0
    dY = np.zeros((Mt, H), np.uint16)
    dY[realrows] = wl.normal_bf16(rng, (real, H), std=2.0 ** -10)
    dH = np.zeros((Mt, I2), np.uint16)        # gradient at gate_up's output
    dH[realrows] = wl.normal_bf16(rng, (real, I2), std=2.0 ** -10)
    Xperm = np.zeros((Mt, H), np.uint16)
    Xperm[realrows] = d["X"][d["row_token"][realrows]]
    t = {"W_gu": _bf16_dev(d["W_gu"], dev), "W_d": _bf16_dev(d["W_d"], dev), "X": _bf16_dev(d["X"], dev),
         "A_d": _bf16_dev(d["A_d"], dev), "dY": _bf16_dev(dY, dev), "dH": _bf16_dev(dH, dev),
         "Xperm": _bf16_dev(Xperm, dev)}
    idx = torch.from_numpy(d["row_token"]).to(dev)
    offs = torch.from_numpy(offs_np).to(dev)
    sizes = np.diff(offs_np.astype(np.int64))
    offs128_np = np.concatenate([[0], np.cumsum(-(-sizes // 128) * 128)]).astype(np.int32)
    T128 = int(offs128_np[-1])
    offs128 = torch.from_numpy(offs128_np).to(dev)
    del d, dY, dH, Xperm
    u8 = dict(dtype=torch.uint8, device=dev)

    def packed(n, k):
        return mx.PackedWeight(torch.empty(mx.packed_bytes(G, n, k, 0), **u8),
                               torch.empty(mx.packed_bytes(G, n, k, 1), **u8), G, n, k)
    P_gu, P_d, P_guT, P_dT = packed(I2, H), packed(H, I), packed(H, I2), packed(I, H)

    def act(k):                                   # a [Mt, k] operand in the packed layout
        return mx.PackedWeight(torch.empty(mx.packed_bytes(1, Mt, k, 0), **u8),
                               torch.empty(mx.packed_bytes(1, Mt, k, 1), **u8), 1, Mt, k)
    xq, h1, dy1, dh1 = act(H), act(I), act(H), act(I2)

    def tok(k):                                   # a token-blocked [k, T128] grid, regrouped (canonical)
        return (torch.empty((k, T128), **u8), torch.empty((k, T128 // 32), **u8))
    h0, dy0, dh0, x0 = tok(I), tok(H), tok(I2), tok(H)
    bf = dict(dtype=torch.bfloat16, device=dev)
    y_gu, y_d = torch.empty((Mt, I2), **bf), torch.empty((Mt, H), **bf)
    g_h, g_x = torch.empty((Mt, I), **bf), torch.empty((Mt, H), **bf)
    dW_d = torch.empty((G, H, I), dtype=torch.float32, device=dev)
    dW_gu = torch.empty((G, I2, H), dtype=torch.float32, device=dev)
    ops = [
        ("w_gu_dual_packed", lambda: mx.quantize_dual_packed_(t["W_gu"], P_gu, P_guT)),
        ("w_d_dual_packed", lambda: mx.quantize_dual_packed_(t["W_d"], P_d, P_dT)),
        ("gather_quantize_X", lambda: mx.quantize_gather_packed_(t["X"], idx, xq)),
        ("fprop_gate_up", lambda: mx.grouped_gemm_packed(xq, P_gu, offs, torch.bfloat16, out=y_gu)),
        ("quantize_dual_h", lambda: mx.quantize_dual_grouped_packed_(t["A_d"], offs, offs128, h0, h1)),
        ("fprop_down", lambda: mx.grouped_gemm_packed(h1, P_d, offs, torch.bfloat16, out=y_d)),
        ("quantize_dual_dY", lambda: mx.quantize_dual_grouped_packed_(t["dY"], offs, offs128, dy0, dy1)),
        ("dgrad_down", lambda: mx.grouped_gemm_packed(dy1, P_dT, offs, torch.bfloat16, out=g_h)),
        ("wgrad_down", lambda: mx.grouped_gemm_wgrad(*dy0, *h0, offs128, torch.float32, out=dW_d)),
        ("quantize_dual_dH", lambda: mx.quantize_dual_grouped_packed_(t["dH"], offs, offs128, dh0, dh1)),
        ("dgrad_gate_up", lambda: mx.grouped_gemm_packed(dh1, P_guT, offs, torch.bfloat16, out=g_x)),
        ("quantize_X_axis0", lambda: mx.quantize_dual_grouped_into(t["Xperm"], offs, offs128, *x0)),
        ("wgrad_gate_up", lambda: mx.grouped_gemm_wgrad(*dh0, *x0, offs128, torch.float32, out=dW_gu)),
    ]
    torch.cuda.synchronize()
    ms, avg = run_timed(ops, args, live=("wgrad_gate_up",))
    # the weight-gradient GEMMs over the 32-padded canonical token grids and
    # over the regrouped grids in the packed layout
    # (mxfp8_grouped_gemm_wgrad_packed), for comparison (operands quantized
    # once, outside the timing)
    p32, pk = {}, {}
    for name, src, cols in (("dY", t["dY"], H), ("h", t["A_d"], I), ("dH", t["dH"], I2), ("X", t["Xperm"], H)):
        p32[name] = (torch.empty((cols, Mt), **u8), torch.empty((cols, Mt // 32), **u8))
        mx.quantize_into(src, 0, *p32[name])
        pk[name] = mx.PackedWeight(torch.empty(mx.packed_bytes(1, cols, T128, 0), **u8),
                                   torch.empty(mx.packed_bytes(1, cols, T128, 1), **u8), 1, cols, T128)
        mx.quantize_dual_grouped_packed_(src, offs, offs128, pk[name])
    cmp_ops = [("wgrad_down_32", lambda: mx.grouped_gemm_wgrad(*p32["dY"], *p32["h"], offs, torch.float32, out=dW_d)),
               ("wgrad_gate_up_32", lambda: mx.grouped_gemm_wgrad(*p32["dH"], *p32["X"], offs, torch.float32,
                                                                   out=dW_gu)),
               ("wgrad_down_packed", lambda: mx.grouped_gemm_wgrad_packed(pk["dY"], pk["h"], offs128, torch.float32,
                                                                           out=dW_d)),
               ("wgrad_gate_up_packed", lambda: mx.grouped_gemm_wgrad_packed(pk["dH"], pk["X"], offs128,
                                                                              torch.float32, out=dW_gu))]
    # the forward and data-gradient grouped GEMMs with A read from the
    # canonical grids of the same rows (mxfp8_grouped_gemm), for comparison
    c1 = {}
    for name, src, w in (("X", None, H), ("h", t["A_d"], I), ("dY", t["dY"], H), ("dH", t["dH"], I2)):
        c1[name] = (mx.quantize_gather(t["X"], idx) if src is None else mx.quantize(src, 1))
    cmp_ops += [
        ("fprop_gate_up_canonical_A", lambda: mx.grouped_gemm(*c1["X"], P_gu, offs, torch.bfloat16, out=y_gu)),
        ("fprop_down_canonical_A", lambda: mx.grouped_gemm(*c1["h"], P_d, offs, torch.bfloat16, out=y_d)),
        ("dgrad_down_canonical_A", lambda: mx.grouped_gemm(*c1["dY"], P_dT, offs, torch.bfloat16, out=g_h)),
        ("dgrad_gate_up_canonical_A", lambda: mx.grouped_gemm(*c1["dH"], P_guT, offs, torch.bfloat16, out=g_x))]
    _, avg32 = run_timed(cmp_ops, argparse.Namespace(steps=max(5, args.steps // 4), warmup=2))
    del p32, c1, pk
    f_gu = 2.0 * real * I2 * H
    f_d = 2.0 * real * H * I
    flops = {"fprop_gate_up": f_gu, "fprop_down": f_d, "dgrad_down": f_d, "wgrad_down": f_d,
             "dgrad_gate_up": f_gu, "wgrad_gate_up": f_gu}
    kern = {}
    for name, us in avg.items():
        if name in flops:
            tf = flops[name] / (us * 1e-6) / 1e12
            kern[name] = {"us": round(us, 2), "TFLOP/s": round(tf, 1), "frac_mxfp8_peak": round(tf / MXFP8_PEAK_TFLOPS, 4)}
        else:
            kern[name] = {"us": round(us, 2)}
    for name, us in avg32.items():
        base, note = ((name[:-3], "32-padded canonical token grids") if name.endswith("_32") else
                      (name[:-len("_packed")], "regrouped token grids in the packed layout") if name.endswith("_packed")
                      else (name[:-len("_canonical_A")], "A from the canonical grid"))
        tf = flops[base] / (us * 1e-6) / 1e12
        kern[name] = {"us": round(us, 2), "TFLOP/s": round(tf, 1), "frac_mxfp8_peak": round(tf / MXFP8_PEAK_TFLOPS, 4),
                      "note": note + ", not part of the step"}
    total = sum(flops.values())
    gemm_us = sum(avg[k] for k in flops)
    return _line("MXFP8 GEMM TFLOP/s (% MX peak) + quantize GB/s (% HBM) at Qwen3-8B shapes",
                 round(total / (ms * 1e-3) / 1e12, 2), "TFLOP/s", args, ms,
                 "mxfp8-e4m3/e8m0, fp32 accumulate, bf16 out (fprop/dgrad), fp32 out (wgrad)",
                 {"workload": "qwen3-30b-a3b MoE expert layer learner micro-batch: 8192 tokens, 128 experts, "
                              "Zipf(1.1) top-8, forward + dgrad + wgrad of gate_up and down",
                  "tokens": 8192, "experts": G, "rows_real": real, "rows_padded": Mt,
                  "wgrad_token_grid_rows": T128},
                 kernels=kern, flops_basis="unpadded rows",
                 summary={"gemm_us": round(gemm_us, 1), "gemm_TFLOP/s": round(total / (gemm_us * 1e-6) / 1e12, 1),
                          "other_us": round(sum(avg.values()) - gemm_us, 1)})


def bench_sync(args, dev):
    """Shared-grid weight sync of Qwen3-8B: quantize along K and repack all 144
    linear weights (36 layers x qkv, o, gate_up, down; 6.95e9 elements).  BF16
    weights are drawn on the device (seeded Philox); one step = the whole sync."""
    import torch
    import mxfp8_block_scaled_05_amd as mx
    import workloads as wl

    layers = wl.QWEN3_8B["layers"]
    tensors = []
    for L in range(layers):
        for j, (name, N, K) in enumerate(wl.sync_layer_shapes()):
            W = wl.torch_normal_bf16((N, K), 0.02, seed=1000 + 4 * L + j, device=dev)
            q = torch.empty((N, K), dtype=torch.uint8, device=dev)
            sc = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
            pk = mx.PackedWeight(torch.empty(mx.packed_bytes(1, N, K, 0), dtype=torch.uint8, device=dev),
                                 torch.empty(mx.packed_bytes(1, N, K, 1), dtype=torch.uint8, device=dev), 1, N, K)
            tensors.append((name, W, q, sc, pk))
    n_elts = sum(W.numel() for _, W, _, _, _ in tensors)
    # the sync: every weight quantized along K into its canonical grid (what a
    # learner sends) and the GEMM's packed layout (what the sampler's graphs
    # read) in one pass per weight
    ops = [("quantize_packed_" + name, lambda W=W, q=q, sc=sc, pk=pk: mx.quantize_packed_(W, pk, q, sc))
           for name, W, q, sc, pk in tensors]
    # the same, up to 32 weights per launch (mxfp8_quantize_packed_many)
    jobs = [(W, pk, q, sc) for _, W, q, sc, pk in tensors]
    many = [("quantize_packed_many_%d" % i, lambda c=jobs[i:i + mx.PACKED_JOBS_MAX]: mx.quantize_packed_many_(c))
            for i in range(0, len(jobs), mx.PACKED_JOBS_MAX)]
    # the same result by quantize + repack, for comparison
    unfused = []
    for name, W, q, sc, pk in tensors:
        unfused.append(("quantize_" + name, lambda W=W, q=q, sc=sc: mx.quantize_into(W, 1, q, sc)))
        unfused.append(("repack_" + name, lambda q=q, sc=sc, pk=pk: mx.repack_(q, sc, pk)))
    torch.cuda.synchronize()
    # eager: one host launch per call (host-bound: 144 launches per sync)
    eager_ms, avg = run_timed(ops, argparse.Namespace(steps=max(2, args.steps // 5), warmup=1))

    def replayed(oplist, steps):
        # recorded once into a HIP graph and replayed, as a sampler replays its
        # captured graphs after writing weights in place
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, fn in oplist:
                fn()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / steps, e0.elapsed_time(e1) / steps

    ms, gpu_ms = replayed(many, args.steps)
    one_ms, one_gpu_ms = replayed(ops, args.steps)
    unf_ms, unf_gpu_ms = replayed(unfused, max(2, args.steps // 2))
    # post-sync self-check of one synchronized layer (layer 0 qkv): serving
    # GEMM on a 128-row N(0,1) probe against the dequantized grid
    _, W0, q0, s0, pk0 = tensors[0]
    mx.selfcheck_rel_err(q0, s0, pk0, seed=1)
    t0 = time.perf_counter()
    rel0 = mx.selfcheck_rel_err(q0, s0, pk0, seed=2)[0]
    check_ms = 1e3 * (time.perf_counter() - t0)
    alg = n_elts * (2 + 2 * (1 + 1 / 32))          # bf16 in; canonical + packed out
    kern = {}
    for name, N, K in wl.sync_layer_shapes():
        kern["quantize_packed_" + name] = _bw(avg["quantize_packed_" + name], N * K * (2 + 2 * (1 + 1 / 32)))
    gbs = alg / (ms * 1e-3) / 1e9
    return _line("weight sync GB/s (% HBM): quantize + repack of all Qwen3-8B linears",
                 round(gbs, 1), "GB/s", args, ms, "bf16 -> mxfp8-e4m3/e8m0",
                 {"workload": "qwen3-8b weight sync: every linear (36 layers x qkv, o, gate_up, down) quantized "
                              "along K into its canonical grid and the packed GEMM layout in one pass, "
                              "32 weights per launch, replayed as one HIP graph",
                  "elements": n_elts},
                 kernels=kern, kernels_note="one launch per weight (mxfp8_quantize_packed): per-call HIP-event times from the eager run (they include "
                                            "host launch gaps when the host falls behind)",
                 summary={"algorithmic_GB": round(alg / 1e9, 2), "graph_gpu_ms": round(gpu_ms, 3),
                          "launches_per_sync": len(many),
                          "one_launch_per_weight_graph_ms": round(one_ms, 3),
                          "eager_ms_per_sync": round(eager_ms, 3),
                          "unfused_quantize_then_repack_ms": round(unf_ms, 3),
                          "selfcheck_qkv_rel_err": round(rel0, 5), "selfcheck_ms": round(check_ms, 3),
                          "unfused_GB_moved": round(n_elts * (Q_BYTES_PER_ELT + REPACK_BYTES_PER_ELT) / 1e9, 2),
                          "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)},
                 roofline={"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                           "kernel": "whole sync (quantize + repack)"})


def bench_sweep(args, dev):
    """One Qwen3-8B decoder layer's four linears at M tokens, MXFP8 (quantize
    the input along K straight into the GEMM's packed operand layout + GEMM
    against packed weights, bf16 out; mxfp8_gemm_packed_splitk with a
    preallocated workspace, which splits K only for shapes with few output
    tiles) against BF16
    (torch.nn.functional.linear -> hipBLASLt).  Fits t = F + c*M per arm, for
    GPU time (events around the four linears) and for host wall time per layer
    call, and reports the break-even M* = dF / dc if it lies in range."""
    import torch
    import torch.nn.functional as F_
    import mxfp8_block_scaled_05_amd as mx
    import workloads as wl

    Ms = [512, 1024, 2048, 3072, 4096, 6144, 8192, 12288, 16384]
    shapes = wl.sync_layer_shapes()
    Wb, P = [], []
    for j, (name, N, K) in enumerate(shapes):
        W = wl.torch_normal_bf16((N, K), 0.02, seed=2000 + j, device=dev)
        w = mx.repack(*mx.quantize(W, 1))
        Wb.append(W)
        P.append(w)
    Xall = {K: wl.torch_normal_bf16((max(Ms), K), 1.0, seed=3000 + K, device=dev) for _, _, K in shapes}
    rows = []
    for M in Ms:
        xs = [Xall[K][:M] for _, _, K in shapes]
        qs = [mx.PackedWeight(torch.empty(mx.packed_bytes(1, M, K, 0), dtype=torch.uint8, device=dev),
                              torch.empty(mx.packed_bytes(1, M, K, 1), dtype=torch.uint8, device=dev), 1, M, K)
              for _, _, K in shapes]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, N, _ in shapes]
        # split-K workspaces for the shapes with few output tiles (allocated
        # here, outside the timing; none where the library would not split)
        wss = [torch.empty(mx.gemm_splitk_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
               for _, N, K in shapes]

        def mx_layer():
            for x, a, w, y, wsp in zip(xs, qs, P, ys, wss):
                mx.quantize_many_layouts_([(x, a)])
                mx.gemm_packed(a, w, torch.bfloat16, out=y, workspace=wsp)

        def bf_layer():
            for x, W, y in zip(xs, Wb, ys):
                torch.mm(x, W.t(), out=y)

        res = {"M": M}
        for arm, fn in (("mxfp8", mx_layer), ("bf16", bf_layer)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            n = 20
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[arm + "_gpu_us"] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
            # host wall time per layer call, no synchronization inside
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            host = time.perf_counter() - t0
            torch.cuda.synchronize()
            res[arm + "_host_us"] = round(host * 1e6 / n, 2)
            # the layer's launches captured once as a HIP graph and replayed:
            # GPU time without any per-launch host dispatch
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(n):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            res[arm + "_graph_us"] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
            del graph
        rows.append(res)

    def fit(key):
        m = np.array([r["M"] for r in rows], np.float64)
        t = np.array([r[key] for r in rows], np.float64)
        c, f = np.polyfit(m, t, 1)
        return f, c

    fits = {}
    for kind in ("gpu", "graph", "host"):
        fm, cm = fit("mxfp8_%s_us" % kind)
        fb, cb = fit("bf16_%s_us" % kind)
        x = (fm - fb) / (cb - cm) if cb != cm else None
        # measured: the sweep points between which the faster arm changes
        faster = [r["mxfp8_%s_us" % kind] < r["bf16_%s_us" % kind] for r in rows]
        measured = [[rows[i]["M"], rows[i + 1]["M"]] for i in range(len(rows) - 1) if faster[i] != faster[i + 1]]
        fits[kind] = {"mxfp8_F_us": round(fm, 2), "mxfp8_c_ns_per_token": round(cm * 1e3, 3),
                      "bf16_F_us": round(fb, 2), "bf16_c_ns_per_token": round(cb * 1e3, 3),
                      "break_even_M": round(x, 0) if x is not None and Ms[0] <= x <= Ms[-1] else None,
                      "fit_crossing_M": round(x, 0) if x is not None else None,
                      "measured_crossings": measured,
                      "mxfp8_faster_at": [r["M"] for r, f in zip(rows, faster) if f]}
    flops_tok = sum(2.0 * N * K for _, N, K in shapes)
    big = rows[-1]
    speedup = big["bf16_gpu_us"] / big["mxfp8_gpu_us"]
    return _line("MXFP8 vs BF16 layer time over M (break-even tokens)", round(speedup, 3),
                 "x speedup of MXFP8 over BF16 GPU time at M=16384", args, 0.0,
                 "mxfp8-e4m3/e8m0 vs bf16, fp32 accumulate, bf16 out",
                 {"workload": "qwen3-8b decoder layer linears (qkv, o, gate_up, down) at M in %s" % Ms,
                  "flops_per_token": flops_tok},
                 sweep=rows, fits=fits)


def _bw(us, nbytes):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_baseline_qkv(min_seconds: float = 10.0):
    """The oracle (plain C; OpenMP over independent output rows) on the same
    qkv step at full size: quantize W and X, pack W, and the fp64 GEMM over
    every row of X.  Whole steps are repeated until at least min_seconds have
    passed (no extrapolation from a partial step); the rate is the mean."""
    import oracle
    import workloads as wl
    oracle._load()
    d = wl.qkv(0)
    M, K = d["X"].shape
    N = d["W"].shape[0]
    t = {"quantize_W": 0.0, "quantize_X": 0.0, "repack_W": 0.0, "gemm": 0.0}
    steps = 0
    while steps == 0 or sum(t.values()) < min_seconds:
        t0 = time.perf_counter()
        wq, ws = oracle.quantize(d["W"], 1)
        t["quantize_W"] += time.perf_counter() - t0
        t0 = time.perf_counter()
        xq, xs = oracle.quantize(d["X"], 1)
        t["quantize_X"] += time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.pack(wq, ws, 1, N, K)
        t["repack_W"] += time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gemm(xq, xs, wq, ws)
        t["gemm"] += time.perf_counter() - t0
        steps += 1
    total = sum(t.values())
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    one = _oracle_single_core()
    return {
        "host": host_description(),
        "single_core": one,
        "value": round(2.0 * M * N * K * steps / total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d full qkv step(s) (quantize W[6144x4096] and X[4096x4096], pack W, "
                  "fp64 GEMM of all 4096 rows), %.1f s in total" % (steps, total),
        "seconds_per_step": {k: round(v / steps, 3) for k, v in t.items()},
    }


def _oracle_single_core_sample():
    """One host thread: the oracle's quantize of W and X and pack of W at full
    size, and its fp64 GEMM over the first 64 rows of X (no extrapolation)."""
    import oracle
    import workloads as wl
    oracle._load()
    d = wl.qkv(0)
    M, K = d["X"].shape
    N = d["W"].shape[0]
    t0 = time.perf_counter()
    wq, ws = oracle.quantize(d["W"], 1)
    xq, xs = oracle.quantize(d["X"], 1)
    tq = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.pack(wq, ws, 1, N, K)
    tp = time.perf_counter() - t0
    rows = np.arange(64)
    t0 = time.perf_counter()
    oracle.gemm(xq, xs, wq, ws, rows=rows)
    tg = time.perf_counter() - t0
    qbytes = (N * K + M * K) * Q_BYTES_PER_ELT
    return {"quantize_GB/s": round(qbytes / tq / 1e9, 3),
            "repack_GB/s": round(N * K * REPACK_BYTES_PER_ELT / tp / 1e9, 3),
            "gemm_GFLOP/s": round(2.0 * rows.size * N * K / tg / 1e9, 3),
            "sample": "quantize W[6144x4096] and X[4096x4096], pack W, fp64 GEMM of 64 rows x 6144 x 4096",
            "seconds": round(tq + tp + tg, 3)}


def _oracle_single_core():
    """_oracle_single_core_sample in a child process limited to one OpenMP
    thread (the child touches no GPU)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = "import json, bench; print(json.dumps(bench._oracle_single_core_sample()))"
    try:
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=300)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None


def secondary_workloads(args, dev):
    """Compact figures of the other configurations, run after the default
    step with few steps each (a few seconds in all): the Qwen3-8B weight sync
    (all 144 linears quantized into the canonical grid and the packed layout),
    the Qwen3-8B MLP learner micro-batch (8192 tokens), and the Qwen3-30B-A3B
    MoE layer forward.  Each is the same code as its --workload line."""
    import torch
    sub = argparse.Namespace(steps=min(args.steps, 10), warmup=min(args.warmup, 2), settle_s=0.1)
    res = {}
    s = bench_sync(sub, dev)
    res["weight_sync"] = {"ms": s["summary"]["graph_gpu_ms"], "GB/s": s["value"],
                          "frac_hbm_peak": s["summary"]["frac_hbm_peak"],
                          "algorithmic_GB": s["summary"]["algorithmic_GB"],
                          "one_launch_per_weight_graph_ms": s["summary"]["one_launch_per_weight_graph_ms"],
                          "what": s["config"]["workload"]}
    gc.collect()
    torch.cuda.empty_cache()
    m = bench_mlp(sub, dev)
    k = m["kernels"]
    res["mlp_step"] = {"ms_per_step": m["ms_per_step"], "TFLOP/s": m["value"],
                       "gemm_TFLOP/s": m["summary"]["gemm_TFLOP/s"],
                       "graph_replay_ms_per_step": m["summary"]["graph_replay_ms_per_step"],
                       "gemms": {g: k[g] for g in k if g.startswith("gemm_")},
                       "canonical_A_gemm_us": m["summary"]["canonical_A_gemm_us"],
                       "quantize": {q: k[q] for q in k if q.startswith("quantize_")},
                       "what": m["config"]["workload"]}
    gc.collect()
    torch.cuda.empty_cache()
    e = bench_moe(sub, dev)
    k = e["kernels"]
    res["moe_forward"] = {"ms_per_step": e["ms_per_step"], "TFLOP/s": e["value"],
                          "grouped_gemm_gate_up": k["grouped_gemm_gate_up"],
                          "grouped_gemm_down": k["grouped_gemm_down"],
                          "what": e["config"]["workload"]}
    gc.collect()
    torch.cuda.empty_cache()
    res["note"] = "steps=%d warmup=%d per workload; HIP-event kernel times as in each --workload line" % (
        sub.steps, sub.warmup)
    return res


def copy_calibration(dev, nbytes: int = 512 << 20, reps: int = 3):
    """A plain device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters of a profiled run (reads nbytes, writes nbytes)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed seconds of the step before the W warm-up steps (clock ramp)")
    ap.add_argument("--workload", default="qkv", choices=["qkv", "mlp", "moe", "moe_train", "sync", "sweep"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="default workload only: skip the compact weight-sync / MLP / MoE figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 512 MiB device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp8_block_scaled_05_amd as mx
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    mx.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(dev)
    if args.workload == "qkv":
        out = bench_qkv(args, dev)
        if not args.no_secondary:
            out["secondary"] = secondary_workloads(args, dev)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_qkv()
    else:
        out = {"mlp": bench_mlp, "moe": bench_moe, "moe_train": bench_moe_train, "sync": bench_sync,
               "sweep": bench_sweep}[args.workload](args, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
