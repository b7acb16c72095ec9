"""MXFP8 oracle -- TEST INFRASTRUCTURE ONLY.

Thin numpy-facing wrappers over ``mxfp8_oracle.c``, a plain scalar fp64 CPU
statement of the MXFP8 codec, quantizer, dequantizer, GEMM over dequantized
operands, grouped GEMM and the packed weight layout.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package; the library under ``mxfp8_block_scaled_05_amd`` never does.

Source of what is computed: "End-to-End MXFP8 RL on Blackwell: What Matching
Buys, When It Pays Off, and How It Fails" (verl blog), section "The pipeline"
(paragraph "The format" and the learner paragraph) and section "Correctness:
how it fails" (post-sync self-check); the encodings are those of the OCP MX
v1.0 specification that the format paragraph cites.  Every function below is
pinned by CPU tests (tests/test_oracle_*.py) against closed forms, library
decoders, brute-force searches, exact integer arithmetic and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libmxfp8_oracle.so")
_lock = threading.Lock()
_lib = None

BLOCK = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over independent outputs)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.mxo_bf16_decode.restype = ctypes.c_double
        lib.mxo_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.mxo_bf16_encode.restype = ctypes.c_uint16
        lib.mxo_bf16_encode.argtypes = [ctypes.c_double]
        lib.mxo_e4m3_decode.restype = ctypes.c_double
        lib.mxo_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.mxo_e8m0_decode.restype = ctypes.c_double
        lib.mxo_e8m0_decode.argtypes = [ctypes.c_uint8]
        lib.mxo_e4m3_encode.restype = ctypes.c_uint8
        lib.mxo_e4m3_encode.argtypes = [ctypes.c_double]
        lib.mxo_e4m3_encode_n.restype = None
        lib.mxo_e4m3_encode_n.argtypes = [P, I64, P]
        lib.mxo_e4m3_decode_n.restype = None
        lib.mxo_e4m3_decode_n.argtypes = [P, I64, P]
        lib.mxo_block_scale.restype = ctypes.c_uint8
        lib.mxo_block_scale.argtypes = [P, I64]
        lib.mxo_quantize.restype = ctypes.c_int
        lib.mxo_quantize.argtypes = [P, I64, I64, ctypes.c_int, P, P]
        for name in ("mxo_dequantize_f64", "mxo_dequantize_f32", "mxo_dequantize_bf16"):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [P, P, I64, I64, ctypes.c_int, P]
        lib.mxo_gemm_rows.restype = ctypes.c_int
        lib.mxo_gemm_rows.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P, P]
        lib.mxo_grouped_gemm_rows.restype = ctypes.c_int
        lib.mxo_grouped_gemm_rows.argtypes = [P, P, P, P, P, I64, I64, I64, I64,
                                              P, I64, P, P, P]
        lib.mxo_packed_bytes.restype = I64
        lib.mxo_packed_bytes.argtypes = [I64, I64, I64, ctypes.c_int]
        lib.mxo_pack.restype = ctypes.c_int
        lib.mxo_pack.argtypes = [P, P, I64, I64, I64, P, P]
        lib.mxo_unpack.restype = ctypes.c_int
        lib.mxo_unpack.argtypes = [P, P, I64, I64, I64, P, P]
        _lib = lib
        return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ scalars

def e4m3_decode(code: int) -> float:
    return _load().mxo_e4m3_decode(code & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(_load().mxo_e4m3_encode(float(v)))


def e8m0_decode(code: int) -> float:
    return _load().mxo_e8m0_decode(code & 0xFF)


def bf16_decode(bits: int) -> float:
    return _load().mxo_bf16_decode(bits & 0xFFFF)


def bf16_encode(v: float) -> int:
    return int(_load().mxo_bf16_encode(float(v)))


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().mxo_e4m3_encode_n(_p(v), v.size, _p(out))
    return out


def e4m3_decode_table() -> np.ndarray:
    """fp64 value of each of the 256 E4M3 codes (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


# ------------------------------------------------------------------ tensors

def block_scale(block_bits: np.ndarray) -> int:
    b = np.ascontiguousarray(block_bits, dtype=np.uint16).reshape(-1)
    assert b.size == BLOCK
    return int(_load().mxo_block_scale(_p(b), 1))


def quantize(x_bits: np.ndarray, axis: int):
    """x_bits: uint16 [rows, cols] BF16 patterns.  Returns (q, scales) as uint8
    arrays: axis=1 -> q[rows, cols], s[rows, cols/32]; axis=0 -> q[cols, rows],
    s[cols, rows/32] (transposed so the block axis is contiguous)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    if axis == 1:
        q = np.empty((rows, cols), np.uint8)
        s = np.empty((rows, cols // BLOCK), np.uint8)
    elif axis == 0:
        q = np.empty((cols, rows), np.uint8)
        s = np.empty((cols, rows // BLOCK), np.uint8)
    else:
        raise ValueError("axis must be 0 or 1")
    rc = _load().mxo_quantize(_p(x), rows, cols, axis, _p(q), _p(s))
    if rc:
        raise ValueError("block axis is not a multiple of 32")
    return q, s


def regroup_rows(x_bits: np.ndarray, src_offsets, dst_offsets, rows_out: int) -> np.ndarray:
    """x' [rows_out, cols]: group g's rows x[src[g]:src[g+1]] placed at rows
    dst[g] .. dst[g] + len_g, zero rows everywhere else (well-formed tables:
    non-decreasing, each destination range at least as long as its source)."""
    x_bits = np.asarray(x_bits, np.uint16)
    src = np.asarray(src_offsets, np.int64)
    dst = np.asarray(dst_offsets, np.int64)
    out = np.zeros((rows_out, x_bits.shape[1]), np.uint16)
    for g in range(src.size - 1):
        n = src[g + 1] - src[g]
        assert n >= 0 and dst[g + 1] - dst[g] >= n and dst[g] + n <= rows_out
        out[dst[g]:dst[g] + n] = x_bits[src[g]:src[g + 1]]
    return out


def quantize_grouped_axis0(x_bits: np.ndarray, src_offsets, dst_offsets, rows_out: int):
    """The token-blocked grid of a token-sorted MoE tensor with every group
    moved to its destination rows: quantize(regroup_rows(x, ...), axis=0)
    (the pad rows are zero, so their blocks get zero codes and scale code 0).
    Follows the learner paragraph of "The pipeline" (token-axis blocks for
    the weight-gradient GEMM, per-expert groups)."""
    return quantize(regroup_rows(x_bits, src_offsets, dst_offsets, rows_out), 0)


def dequantize(q: np.ndarray, s: np.ndarray, rows: int, cols: int, axis: int,
               dtype: str = "f64") -> np.ndarray:
    """Inverse of ``quantize``: [rows, cols] in the original orientation.
    dtype 'f64' (exact), 'f32' (RNE from fp64) or 'bf16' (uint16 bits, RNE)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    lib = _load()
    if dtype == "f64":
        out = np.empty((rows, cols), np.float64)
        lib.mxo_dequantize_f64(_p(q), _p(s), rows, cols, axis, _p(out))
    elif dtype == "f32":
        out = np.empty((rows, cols), np.float32)
        lib.mxo_dequantize_f32(_p(q), _p(s), rows, cols, axis, _p(out))
    elif dtype == "bf16":
        out = np.empty((rows, cols), np.uint16)
        lib.mxo_dequantize_bf16(_p(q), _p(s), rows, cols, axis, _p(out))
    else:
        raise ValueError(dtype)
    return out


def gemm(a_q, a_s, b_q, b_s, rows=None):
    """C_ref = A' B'^T and S = |A'| |B'|^T (fp64) over dequantized K-contiguous
    operands A[M,K], B[N,K]; only the given rows of A when ``rows`` is set.
    Returns (c_ref, c_abs) of shape [len(rows) or M, N]."""
    a_q = np.ascontiguousarray(a_q, np.uint8)
    a_s = np.ascontiguousarray(a_s, np.uint8)
    b_q = np.ascontiguousarray(b_q, np.uint8)
    b_s = np.ascontiguousarray(b_s, np.uint8)
    M, K = a_q.shape
    N = b_q.shape[0]
    assert b_q.shape[1] == K and a_s.shape == (M, K // BLOCK) and b_s.shape == (N, K // BLOCK)
    if rows is None:
        idx = np.arange(M, dtype=np.int64)
    else:
        idx = np.ascontiguousarray(rows, np.int64)
    c = np.empty((idx.size, N), np.float64)
    sabs = np.empty((idx.size, N), np.float64)
    rc = _load().mxo_gemm_rows(_p(a_q), _p(a_s), _p(b_q), _p(b_s), M, N, K,
                               _p(idx), idx.size, _p(c), _p(sabs))
    if rc:
        raise RuntimeError("oracle gemm failed: %d" % rc)
    return c, sabs


def grouped_gemm(a_q, a_s, b_q, b_s, offsets, rows=None):
    """Per-expert GEMM: rows [off[g], off[g+1]) of A times B_g^T, with B given
    canonically as [G, N, K] / [G, N, K/32].  Returns (c_ref, c_abs, group)
    for the requested rows; group is -1 for rows in no group (their c is
    undefined)."""
    a_q = np.ascontiguousarray(a_q, np.uint8)
    a_s = np.ascontiguousarray(a_s, np.uint8)
    b_q = np.ascontiguousarray(b_q, np.uint8)
    b_s = np.ascontiguousarray(b_s, np.uint8)
    off = np.ascontiguousarray(offsets, np.int32)
    M, K = a_q.shape
    G, N, K2 = b_q.shape
    assert K2 == K and off.size == G + 1
    idx = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    c = np.zeros((idx.size, N), np.float64)
    sabs = np.zeros((idx.size, N), np.float64)
    grp = np.empty(idx.size, np.int32)
    rc = _load().mxo_grouped_gemm_rows(_p(a_q), _p(a_s), _p(b_q), _p(b_s), _p(off),
                                       G, M, N, K, _p(idx), idx.size, _p(c),
                                       _p(sabs), _p(grp))
    if rc:
        raise RuntimeError("oracle grouped gemm failed: %d" % rc)
    return c, sabs, grp


def packed_bytes(batch: int, N: int, K: int, which: int) -> int:
    return int(_load().mxo_packed_bytes(batch, N, K, which))


def pack(q, s, batch, N, K):
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    qp = np.empty(packed_bytes(batch, N, K, 0), np.uint8)
    sp = np.empty(packed_bytes(batch, N, K, 1), np.uint8)
    if _load().mxo_pack(_p(q), _p(s), batch, N, K, _p(qp), _p(sp)):
        raise ValueError("bad pack arguments")
    return qp, sp


def unpack(qp, sp, batch, N, K):
    qp = np.ascontiguousarray(qp, np.uint8)
    sp = np.ascontiguousarray(sp, np.uint8)
    q = np.empty((batch, N, K), np.uint8)
    s = np.empty((batch, N, K // BLOCK), np.uint8)
    if _load().mxo_unpack(_p(qp), _p(sp), batch, N, K, _p(q), _p(s)):
        raise ValueError("bad unpack arguments")
    return q, s


def gemm_bound_ok(c_dev: np.ndarray, c_ref: np.ndarray, c_abs: np.ndarray,
                  out_dtype: str = "f32", rel: float = 1e-4):
    """Element-wise acceptance test of a device GEMM result.

    fp32 output: |C - C_ref| <= rel * sum_k |a_k b_k|.
    bf16 output: the same plus the bf16 rounding of the result,
    2^-8 * |C_ref| (half an ulp of an 8-bit significand, relative).
    Returns (ok, worst ratio of error to allowance)."""
    c_dev = np.asarray(c_dev, np.float64)
    allow = rel * c_abs
    if out_dtype == "bf16":
        allow = allow + np.abs(c_ref) * 2.0 ** -8
    err = np.abs(c_dev - c_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allow > 0, err / np.where(allow > 0, allow, 1), np.where(err > 0, np.inf, 0.0))
    ok = bool(np.all(err <= allow)) and bool(np.all(np.isfinite(c_dev)))
    return ok, float(np.max(ratio)) if ratio.size else 0.0
