"""Benchmark of the MXFP8 hot path on one MI355X.

Default step (the Qwen3-8B qkv_proj layer, 4096 tokens): quantize W[6144x4096]
and X[4096x4096] along K, repack W into the GEMM layout, and run the MXFP8
GEMM Y = X W^T with bf16 output.  Inputs are resident in HBM before the timed
region; R input/output sets are rotated so the working set (> 512 MB) does not
sit in the 256 MB Infinity Cache.  Every kernel launch is bracketed by HIP
events on the stream it runs on, so each kernel's average duration is
measured live; `value` is the whole step's throughput (2MNK / step time).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload qkv|mlp|moe|sync|sweep]
                    [--no-cpu-baseline]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
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

    def reset(self):
        self.pending = {}


def bench_qkv(args, dev):
    import torch
    import mxfp8_block_scaled_05_amd as mx
    import workloads as wl

    M, K = 4096, wl.QWEN3_8B["hidden"]
    N = wl.QWEN3_8B["qkv"]
    d = wl.qkv(0, tokens=M)
    per_set = (N * K + M * K) * 2 + (N * K + M * K) + N * K + M * N * 2
    R = max(2, int(np.ceil(600e6 / per_set)))
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
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        sets.append((X, W, xq, xs, wq, ws, w, y))
    torch.cuda.synchronize()
    timer = KernelTimer()

    def step(i, timed):
        X, W, xq, xs, wq, ws, w, y = sets[i % R]
        if timed:
            timer.time("quantize_W", lambda: mx.quantize_into(W, 1, wq, ws))
            timer.time("quantize_X", lambda: mx.quantize_into(X, 1, xq, xs))
            timer.time("repack_W", lambda: mx.repack_(wq, ws, w))
            timer.time("gemm", lambda: mx.gemm(xq, xs, w, torch.bfloat16, out=y))
        else:
            mx.quantize_into(W, 1, wq, ws)
            mx.quantize_into(X, 1, xq, xs)
            mx.repack_(wq, ws, w)
            mx.gemm(xq, xs, w, torch.bfloat16, out=y)

    for i in range(args.warmup):
        step(i, True)
    torch.cuda.synchronize()
    timer.reset()
    # timed region: K steps, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = timer.averages_us()
    ms_per_step = 1e3 * wall / args.steps
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (avg["gemm"] * 1e-6) / 1e12
    kern = {
        "quantize_W": _bw(avg["quantize_W"], N * K * Q_BYTES_PER_ELT),
        "quantize_X": _bw(avg["quantize_X"], M * K * Q_BYTES_PER_ELT),
        "repack_W": _bw(avg["repack_W"], N * K * REPACK_BYTES_PER_ELT),
        "gemm": {"us": round(avg["gemm"], 2), "TFLOP/s": round(gemm_tflops, 1),
                 "frac_mxfp8_peak": round(gemm_tflops / MXFP8_PEAK_TFLOPS, 4)},
    }
    out = {
        "metric": "MXFP8 GEMM TFLOP/s (% MX peak) + quantize GB/s (% HBM) at Qwen3-8B shapes",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3/e8m0, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded N(0,1) activations with 1% x20 outliers, N(0,0.02) weights)",
        "config": {"workload": "qwen3-8b qkv_proj: quantize W[6144x4096] + X[4096x4096] along K, "
                               "repack W, MXFP8 GEMM -> bf16",
                   "M": M, "N": N, "K": K, "rotated_sets": R},
        "kernels": kern,
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": MXFP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / MXFP8_PEAK_TFLOPS, 4),
                     "traffic": measured_gemm_traffic()},
    }
    return out


def _bw(us, nbytes):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_baseline_qkv():
    """The oracle (plain C; OpenMP over independent output rows) on the same
    qkv step at full size: quantize W and X, pack W, and the fp64 GEMM over
    every row of X.  No extrapolation: the whole step is run once."""
    import oracle
    import workloads as wl
    oracle._load()
    d = wl.qkv(0)
    M, K = d["X"].shape
    N = d["W"].shape[0]
    t = {}
    t0 = time.perf_counter()
    wq, ws = oracle.quantize(d["W"], 1)
    t["quantize_W"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    xq, xs = oracle.quantize(d["X"], 1)
    t["quantize_X"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.pack(wq, ws, 1, N, K)
    t["repack_W"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gemm(xq, xs, wq, ws)
    t["gemm"] = time.perf_counter() - t0
    total = sum(t.values())
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": round(2.0 * M * N * K / total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "one full qkv step (quantize W[6144x4096] and X[4096x4096], pack W, "
                  "fp64 GEMM of all 4096 rows) run once",
        "seconds": {k: round(v, 3) for k, v in t.items()},
    }


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qkv", choices=["qkv"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    out = bench_qkv(args, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_qkv()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
