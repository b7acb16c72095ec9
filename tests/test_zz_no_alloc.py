"""The allocation-free split-K GEMM (mxfp8_gemm_splitk_noalloc), called
through the C ABI: its output equals mxfp8_gemm_splitk's with a caller
workspace bit for bit (same plan, same kernels) and lies within the oracle's
bound, on two calls in a row, the second with a smaller input (the static
scratch keeps the first call's partials, which must not leak into it)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from conftest import sample_rows, to_dev, to_host

pytestmark = pytest.mark.gpu

MXFP8_PACKED, MXFP8_CANONICAL = 1, 0


def _say(*a):
    print("no-alloc case:", *a, flush=True)


def _operands(oracle_mod, M, N, K, seed):
    rng = np.random.default_rng(seed)
    xq, xs = oracle_mod.quantize(wl.normal_bf16(rng, (M, K)), 1)
    wq, ws = oracle_mod.quantize(wl.normal_bf16(rng, (N, K), std=0.02), 1)
    return xq, xs, wq, ws


def _noalloc(mx, a_q, a_s, b_q, b_s, layout, M, N, K, out):
    L = mx.lib()
    code = 0 if out.dtype == torch.float32 else 1
    st = L.mxfp8_gemm_splitk_noalloc(ctypes.c_void_p(a_q.data_ptr()), ctypes.c_void_p(a_s.data_ptr()),
                                     ctypes.c_void_p(b_q.data_ptr()), ctypes.c_void_p(b_s.data_ptr()),
                                     layout, M, N, K, ctypes.c_void_p(out.data_ptr()), code,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


# the first shape's plan fills the static scratch exactly (4 slices of
# 512 x 4096 fp32 partials = 32 MiB); the second is smaller; the third does
# not split (plain GEMM path)
CASES = [(512, 4096, 12288, torch.bfloat16, True), (64, 2048, 4096, torch.float32, False),
         (2048, 4096, 1024, torch.bfloat16, True)]


def test_noalloc_splitk_matches_workspace_call(mx, oracle_mod):
    for i, (M, N, K, dt, packed) in enumerate(CASES):
        _say(M, N, K, dt, "packed" if packed else "canonical",
             "workspace bytes", mx.gemm_splitk_workspace_bytes(M, N, K))
        xq, xs, wq, ws = _operands(oracle_mod, M, N, K, 50 + i)
        a_q, a_s = to_dev(xq), to_dev(xs)
        if packed:
            w = mx.repack(to_dev(wq), to_dev(ws))
            b_q, b_s, layout, b = w.q, w.s, MXFP8_PACKED, w
        else:
            b_q, b_s, layout = to_dev(wq), to_dev(ws), MXFP8_CANONICAL
            b = (b_q, b_s)
        ref = mx.gemm(a_q, a_s, b, dt, split_k=True)          # caller workspace through torch
        out = torch.full((M, N), float("nan"), dtype=dt, device=a_q.device)
        assert _noalloc(mx, a_q, a_s, b_q, b_s, layout, M, N, K, out) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (M, N, K)
        rows = sample_rows(M, 256, 64, 60 + i)
        c_ref, c_abs = oracle_mod.gemm(xq, xs, wq, ws, rows=rows)
        got = to_host(out.float())[rows]
        ok, worst = oracle_mod.gemm_bound_ok(got, c_ref, c_abs, "f32" if dt == torch.float32 else "bf16")
        assert ok, worst
    assert mx.gemm_splitk_workspace_bytes(512, 4096, 12288) == 32 << 20
    assert mx.gemm_splitk_workspace_bytes(2048, 4096, 1024) == 0


def test_noalloc_argument_errors(mx):
    L = mx.lib()
    t = torch.empty(64, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    q = ctypes.c_void_p(t.data_ptr() + 1)
    assert L.mxfp8_gemm_splitk_noalloc(None, p, p, p, 1, 4, 4, 64, p, 0, None) == 1
    assert L.mxfp8_gemm_splitk_noalloc(p, p, p, p, 1, 4, 4, 48, p, 0, None) == 2
    assert L.mxfp8_gemm_splitk_noalloc(p, p, p, p, 3, 4, 4, 64, p, 0, None) == 4
    assert L.mxfp8_gemm_splitk_noalloc(p, q, p, p, 1, 4, 4, 64, p, 0, None) == 5
