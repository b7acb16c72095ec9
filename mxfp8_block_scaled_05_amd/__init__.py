"""MI355X (gfx950) MXFP8 library -- Python binding.

Argument marshalling only: every step runs in the HIP kernels of
``libmxfp8.so`` through the C ABI declared in ``include/mxfp8.h``.  PyTorch
supplies device memory and the current stream.  There is no fallback: if the
library is not built, or the device is not gfx950, every call raises.

    q, s   = quantize(x_bf16, axis)                  # E4M3 + E8M0
    x'     = dequantize(q, s, rows, cols, axis, torch.float32 | torch.bfloat16)
    w      = repack(q, s)                            # PackedWeight (kernel layout)
    repack_(q, s, w)                                 # in place, after every update
    c      = gemm(a_q, a_s, w_or_(b_q, b_s), out_dtype)
    c      = grouped_gemm(a_q, a_s, w_experts, d_offsets, out_dtype)
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import torch

__all__ = ["lib", "quantize", "quantize_into", "dequantize", "packed_bytes", "PackedWeight",
           "repack", "repack_", "quantize_packed_axis0_", "quantize_many_", "quantize_packed_many_", "gemm", "grouped_gemm", "grouped_gemm_packed", "MXFP8Error", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp8.so")

MXFP8_F32, MXFP8_BF16 = 0, 1
MXFP8_CANONICAL, MXFP8_PACKED = 0, 1

_lock = threading.Lock()
_lib = None


class MXFP8Error(RuntimeError):
    pass


def lib():
    """Load libmxfp8.so (built in-tree by ``python -m mxfp8_block_scaled_05_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise MXFP8Error("libmxfp8.so is not built (%s); run "
                             "`python -m mxfp8_block_scaled_05_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mxfp8_quantize.argtypes = [P, I64, I64, I32, P, P, P]
        L.mxfp8_dequantize.argtypes = [P, P, I64, I64, I32, P, I32, P]
        L.mxfp8_packed_bytes.argtypes = [I64, I64, I64, I32]
        L.mxfp8_packed_bytes.restype = ctypes.c_size_t
        L.mxfp8_repack.argtypes = [P, P, I64, I64, I64, P, P, P]
        L.mxfp8_gemm.argtypes = [P, P, P, P, I32, I64, I64, I64, P, I32, P]
        L.mxfp8_grouped_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, I32, P]
        L.mxfp8_selfcheck_workspace_bytes.argtypes = [I64, I64, I64]
        L.mxfp8_selfcheck_workspace_bytes.restype = ctypes.c_size_t
        L.mxfp8_selfcheck.argtypes = [P, I64, I64, I64, P, P, P, P, P, P, P]
        L.mxfp8_selfcheck.restype = I32
        L.mxfp8_quantize_batched.argtypes = [P, I64, I64, I64, I32, P, P, P]
        L.mxfp8_quantize_gather.argtypes = [P, I64, I64, P, I64, P, P, P]
        L.mxfp8_quantize_gather_packed.argtypes = [P, I64, I64, P, I64, P, P, P]
        L.mxfp8_quantize_gather_packed.restype = I32
        L.mxfp8_grouped_gemm_wgrad.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, I32, P]
        L.mxfp8_grouped_gemm_wgrad_packed.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, I32, P]
        L.mxfp8_grouped_gemm_wgrad_packed.restype = I32
        for f in ("mxfp8_quantize_batched", "mxfp8_quantize_gather", "mxfp8_grouped_gemm_wgrad"):
            getattr(L, f).restype = I32
        L.mxfp8_quantize_dual.argtypes = [P, I64, I64, P, P, P, P, P]
        L.mxfp8_quantize_dual_grouped.argtypes = [P, I64, I64, P, P, P, P, P, P, I64, I64, P]
        L.mxfp8_quantize_dual_grouped_packed.argtypes = [P, I64, I64, P, P, P, P, I32, P, P, I64, I64, P]
        L.mxfp8_quantize_dual_grouped_packed.restype = I32
        L.mxfp8_gemm_splitk.argtypes = [P, P, P, P, I32, I64, I64, I64, P, I32, P, ctypes.c_size_t, P]
        L.mxfp8_gemm_splitk.restype = I32
        L.mxfp8_gemm_accurate.argtypes = [P, P, P, P, I32, I64, I64, I64, P, I32, P]
        L.mxfp8_gemm_accurate.restype = I32
        L.mxfp8_gemm_packed.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P]
        L.mxfp8_gemm_packed.restype = I32
        L.mxfp8_gemm_packed_splitk.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P, ctypes.c_size_t, P]
        L.mxfp8_gemm_packed_splitk.restype = I32
        L.mxfp8_grouped_gemm_packed.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, I32, P]
        L.mxfp8_grouped_gemm_packed.restype = I32
        L.mxfp8_quantize_dual_packed.argtypes = [P, I64, I64, I64, P, P, P, P, P]
        L.mxfp8_quantize_dual_packed.restype = I32
        L.mxfp8_quantize_many_layouts.argtypes = [P, I64, P]
        L.mxfp8_quantize_many_layouts.restype = I32
        L.mxfp8_gemm_splitk_noalloc.argtypes = [P, P, P, P, I32, I64, I64, I64, P, I32, P]
        L.mxfp8_gemm_splitk_noalloc.restype = I32
        L.mxfp8_gemm_splitk_workspace_bytes.argtypes = [I64, I64, I64]
        L.mxfp8_gemm_splitk_workspace_bytes.restype = ctypes.c_size_t
        L.mxfp8_quantize_packed.argtypes = [P, I64, I64, I64, P, P, P, P, P]
        L.mxfp8_quantize_packed_axis0.argtypes = [P, I64, I64, I64, P, P, P]
        L.mxfp8_quantize_packed_axis0.restype = I32
        L.mxfp8_quantize_many.argtypes = [ctypes.POINTER(QuantJob), I64, P]
        L.mxfp8_quantize_many.restype = I32
        L.mxfp8_quantize_packed_many.argtypes = [ctypes.POINTER(PackedJob), I64, P]
        L.mxfp8_quantize_packed_many.restype = I32
        for f in ("mxfp8_quantize", "mxfp8_dequantize", "mxfp8_repack", "mxfp8_gemm",
                  "mxfp8_grouped_gemm", "mxfp8_quantize_dual", "mxfp8_quantize_packed",
                  "mxfp8_quantize_dual_grouped"):
            getattr(L, f).restype = I32
        L.mxfp8_status_string.argtypes = [I32]
        L.mxfp8_status_string.restype = ctypes.c_char_p
        L.mxfp8_last_hip_error.restype = I32
        L.mxfp8_version.restype = ctypes.c_char_p
        _lib = L
        return L


class QuantJob(ctypes.Structure):
    """One entry of mxfp8_quantize_many's host array (mxfp8_quant_job)."""
    _fields_ = [("x_bf16", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


QUANT_JOBS_MAX = 8


class QuantLayoutJob(ctypes.Structure):
    """mxfp8_quant_layout_job"""
    _fields_ = [("x_bf16", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("layout", ctypes.c_int32), ("q", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class PackedJob(ctypes.Structure):
    """One entry of mxfp8_quantize_packed_many's host array (mxfp8_packed_job)."""
    _fields_ = [("w_bf16", ctypes.c_void_p), ("batch", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("q", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("q_packed", ctypes.c_void_p), ("scales_packed", ctypes.c_void_p)]


PACKED_JOBS_MAX = 32


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        msg = L.mxfp8_status_string(status).decode()
        if status == 6:
            msg += " (hipError %d)" % L.mxfp8_last_hip_error()
        raise MXFP8Error("%s: %s" % (what, msg))


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _out_code(dtype):
    if dtype == torch.float32:
        return MXFP8_F32
    if dtype == torch.bfloat16:
        return MXFP8_BF16
    raise TypeError("output dtype must be torch.float32 or torch.bfloat16")


# ------------------------------------------------------------------ quantize

def quantize_into(x: torch.Tensor, axis: int, q: torch.Tensor, s: torch.Tensor) -> None:
    _need(x, torch.bfloat16, "x")
    _need(q, torch.uint8, "q")
    _need(s, torch.uint8, "scales")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    want_q = (rows, cols) if axis == 1 else (cols, rows)
    want_s = (rows, cols // 32) if axis == 1 else (cols, rows // 32)
    if tuple(q.shape) != want_q or tuple(s.shape) != want_s:
        raise ValueError("q/scales shapes %s/%s, expected %s/%s" % (tuple(q.shape), tuple(s.shape),
                                                                  want_q, want_s))
    _check(lib().mxfp8_quantize(_ptr(x), rows, cols, axis, _ptr(q), _ptr(s), _stream(x.device)),
           "mxfp8_quantize")


def quantize(x: torch.Tensor, axis: int = 1):
    """BF16 [rows, cols] -> (q uint8, scales uint8).  axis=1: q[rows, cols],
    s[rows, cols/32].  axis=0: transposed, q[cols, rows], s[cols, rows/32]."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    if axis == 1:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, max(cols // 32, 0)), dtype=torch.uint8, device=x.device)
    elif axis == 0:
        q = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
        s = torch.empty((cols, max(rows // 32, 0)), dtype=torch.uint8, device=x.device)
    else:
        raise ValueError("axis must be 0 or 1")
    if (axis == 1 and cols % 32) or (axis == 0 and rows % 32):
        raise ValueError("the block axis must be a multiple of 32")
    quantize_into(x, axis, q, s)
    return q, s


def quantize_batched(x: torch.Tensor, axis: int = 1):
    """BF16 [batch, rows, cols] -> (q, s) per matrix as quantize(x[b], axis):
    axis 1: q[batch, rows, cols], s[batch, rows, cols/32]; axis 0 (transposed
    per matrix): q[batch, cols, rows], s[batch, cols, rows/32]."""
    _need(x, torch.bfloat16, "x")
    if x.dim() != 3:
        raise ValueError("x must be 3-D [batch, rows, cols]")
    batch, rows, cols = x.shape
    if axis == 1:
        q = torch.empty((batch, rows, cols), dtype=torch.uint8, device=x.device)
        s = torch.empty((batch, rows, cols // 32), dtype=torch.uint8, device=x.device)
    elif axis == 0:
        q = torch.empty((batch, cols, rows), dtype=torch.uint8, device=x.device)
        s = torch.empty((batch, cols, rows // 32), dtype=torch.uint8, device=x.device)
    else:
        raise ValueError("axis must be 0 or 1")
    _check(lib().mxfp8_quantize_batched(_ptr(x), batch, rows, cols, axis, _ptr(q), _ptr(s),
                                        _stream(x.device)), "mxfp8_quantize_batched")
    return q, s


def quantize_gather_into(x: torch.Tensor, row_index: torch.Tensor, q: torch.Tensor,
                         s: torch.Tensor) -> None:
    """q/s = quantize(x[row_index], 1), rows whose index is outside [0, rows) zero."""
    _need(x, torch.bfloat16, "x")
    _need(row_index, torch.int64, "row_index")
    _need(q, torch.uint8, "q")
    _need(s, torch.uint8, "scales")
    rows_in, cols = x.shape
    rows_out = row_index.numel()
    if tuple(q.shape) != (rows_out, cols) or tuple(s.shape) != (rows_out, cols // 32):
        raise ValueError("q/scales must be [rows_out, cols] / [rows_out, cols/32]")
    _check(lib().mxfp8_quantize_gather(_ptr(x), rows_in, cols, _ptr(row_index), rows_out, _ptr(q),
                                       _ptr(s), _stream(x.device)), "mxfp8_quantize_gather")


def quantize_gather_packed_(x: torch.Tensor, row_index: torch.Tensor, out: "PackedWeight") -> None:
    """mxfp8_quantize_gather_packed: quantize(x[row_index], 1) straight into
    out = PackedWeight(batch 1, N = rows_out, K = cols); rows whose index is
    outside [0, rows) zero."""
    _need(x, torch.bfloat16, "x")
    _need(row_index, torch.int64, "row_index")
    rows_in, cols = x.shape
    rows_out = row_index.numel()
    if not isinstance(out, PackedWeight) or (out.batch, out.N, out.K) != (1, rows_out, cols):
        raise ValueError("out must be PackedWeight(batch 1, N = %d, K = %d)" % (rows_out, cols))
    _need(out.q, torch.uint8, "out.q")
    _need(out.s, torch.uint8, "out.s")
    if out.q.numel() < packed_bytes(1, rows_out, cols, 0) or out.s.numel() < packed_bytes(1, rows_out, cols, 1):
        raise ValueError("out buffers too small")
    _check(lib().mxfp8_quantize_gather_packed(_ptr(x), rows_in, cols, _ptr(row_index), rows_out, _ptr(out.q),
                                              _ptr(out.s), _stream(x.device)), "mxfp8_quantize_gather_packed")


def quantize_gather(x: torch.Tensor, row_index: torch.Tensor):
    rows_out, cols = row_index.numel(), x.shape[1]
    q = torch.empty((rows_out, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows_out, cols // 32), dtype=torch.uint8, device=x.device)
    quantize_gather_into(x, row_index, q, s)
    return q, s


def quantize_dual_into(x: torch.Tensor, q_row: torch.Tensor, s_row: torch.Tensor,
                       q_col: torch.Tensor, s_col: torch.Tensor) -> None:
    """Both grids of x from one read: (q_row, s_row) = quantize(x, 1),
    (q_col, s_col) = quantize(x, 0)."""
    _need(x, torch.bfloat16, "x")
    for t, n in ((q_row, "q_row"), (s_row, "s_row"), (q_col, "q_col"), (s_col, "s_col")):
        _need(t, torch.uint8, n)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    if rows % 32 or cols % 32:
        raise ValueError("rows and cols must be multiples of 32")
    want = ((rows, cols), (rows, cols // 32), (cols, rows), (cols, rows // 32))
    got = tuple(tuple(t.shape) for t in (q_row, s_row, q_col, s_col))
    if got != want:
        raise ValueError("output shapes %s, expected %s" % (got, want))
    _check(lib().mxfp8_quantize_dual(_ptr(x), rows, cols, _ptr(q_row), _ptr(s_row), _ptr(q_col),
                                     _ptr(s_col), _stream(x.device)), "mxfp8_quantize_dual")


def quantize_dual(x: torch.Tensor):
    """BF16 [rows, cols] -> (q_row, s_row, q_col, s_col), the axis-1 and the
    (transposed) axis-0 grids, from one read of x."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    out = (torch.empty((rows, cols), dtype=torch.uint8, device=x.device),
           torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device),
           torch.empty((cols, rows), dtype=torch.uint8, device=x.device),
           torch.empty((cols, rows // 32), dtype=torch.uint8, device=x.device))
    quantize_dual_into(x, *out)
    return out


def quantize_dual_packed_(x: torch.Tensor, row_out: "PackedWeight", col_out: "PackedWeight") -> None:
    """mxfp8_quantize_dual_packed: BF16 [(batch,) rows, cols] -> the packed
    layouts of its axis-1 grids (row_out: PackedWeight(batch, N = rows,
    K = cols)) and of its axis-0 grids (col_out: N = cols, K = rows), from
    one read of x."""
    _need(x, torch.bfloat16, "x")
    if x.dim() not in (2, 3):
        raise ValueError("x must be [rows, cols] or [batch, rows, cols]")
    batch = x.shape[0] if x.dim() == 3 else 1
    rows, cols = x.shape[-2:]
    for t, (n, k), name in ((row_out, (rows, cols), "row_out"), (col_out, (cols, rows), "col_out")):
        if not isinstance(t, PackedWeight) or (t.batch, t.N, t.K) != (batch, n, k):
            raise ValueError("%s must be PackedWeight(batch %d, N = %d, K = %d)" % (name, batch, n, k))
        _need(t.q, torch.uint8, name + ".q")
        _need(t.s, torch.uint8, name + ".s")
        if t.q.numel() < packed_bytes(batch, n, k, 0) or t.s.numel() < packed_bytes(batch, n, k, 1):
            raise ValueError("%s buffers too small" % name)
    _check(lib().mxfp8_quantize_dual_packed(_ptr(x), batch, rows, cols, _ptr(row_out.q), _ptr(row_out.s),
                                            _ptr(col_out.q), _ptr(col_out.s), _stream(x.device)),
           "mxfp8_quantize_dual_packed")


def quantize_dual_grouped_into(x: torch.Tensor, src_offsets: torch.Tensor, dst_offsets: torch.Tensor,
                               q_col: torch.Tensor, s_col: torch.Tensor, q_row: torch.Tensor | None = None,
                               s_row: torch.Tensor | None = None) -> None:
    """(q_row, s_row) = quantize(x, 1) if given; (q_col, s_col) = quantize(x', 0)
    where x' [rows_out, cols] holds group g's rows of x (src_offsets) at
    dst_offsets[g] and zero rows elsewhere.  Offsets: int32 device tensors
    [G+1]; rows_out = q_col.shape[1]."""
    _need(x, torch.bfloat16, "x")
    for t, n in ((q_col, "q_col"), (s_col, "s_col")):
        _need(t, torch.uint8, n)
    if (q_row is None) != (s_row is None):
        raise ValueError("give both q_row and s_row or neither")
    for t, n in ((src_offsets, "src_offsets"), (dst_offsets, "dst_offsets")):
        _need(t, torch.int32, n)
    if x.dim() != 2 or q_col.dim() != 2:
        raise ValueError("x and q_col must be 2-D")
    rows, cols = x.shape
    rows_out = q_col.shape[1]
    G = src_offsets.numel() - 1
    if G < 1 or dst_offsets.numel() != G + 1:
        raise ValueError("src_offsets and dst_offsets must both hold G+1 >= 2 entries")
    if rows % 32 or cols % 32 or rows_out % 32:
        raise ValueError("rows, cols and rows_out must be multiples of 32")
    want = [((cols, rows_out), q_col), ((cols, rows_out // 32), s_col)]
    if q_row is not None:
        _need(q_row, torch.uint8, "q_row")
        _need(s_row, torch.uint8, "s_row")
        want += [((rows, cols), q_row), ((rows, cols // 32), s_row)]
    for shape, t in want:
        if tuple(t.shape) != shape:
            raise ValueError("output shape %s, expected %s" % (tuple(t.shape), shape))
    _check(lib().mxfp8_quantize_dual_grouped(
        _ptr(x), rows, cols, _ptr(q_row) if q_row is not None else None,
        _ptr(s_row) if s_row is not None else None, _ptr(q_col), _ptr(s_col), _ptr(src_offsets),
        _ptr(dst_offsets), G, rows_out, _stream(x.device)), "mxfp8_quantize_dual_grouped")


def quantize_dual_grouped_packed_(x: torch.Tensor, src_offsets: torch.Tensor, dst_offsets: torch.Tensor,
                                  col_out, row_out: "PackedWeight | None" = None) -> None:
    """mxfp8_quantize_dual_grouped_packed: the regrouped token-blocked grid
    of quantize_dual_grouped_into into col_out -- a (q_col [cols, rows_out],
    s_col [cols, rows_out/32]) pair (canonical) or PackedWeight(batch 1,
    N = cols, K = rows_out) (packed) -- and (if given) quantize(x, 1)
    straight into row_out = PackedWeight(batch 1, N = rows, K = cols)."""
    _need(x, torch.bfloat16, "x")
    for t, n in ((src_offsets, "src_offsets"), (dst_offsets, "dst_offsets")):
        _need(t, torch.int32, n)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    G = src_offsets.numel() - 1
    if G < 1 or dst_offsets.numel() != G + 1:
        raise ValueError("src_offsets and dst_offsets must both hold G+1 >= 2 entries")
    outs = []
    if isinstance(col_out, PackedWeight):
        if col_out.batch != 1 or col_out.N != cols:
            raise ValueError("col_out must be PackedWeight(batch 1, N = %d, K = rows_out)" % cols)
        rows_out, layout, qc, sc = col_out.K, MXFP8_PACKED, col_out.q, col_out.s
        outs.append((col_out, (cols, rows_out), "col_out"))
    else:
        qc, sc = col_out
        _need(qc, torch.uint8, "q_col")
        _need(sc, torch.uint8, "s_col")
        if qc.dim() != 2:
            raise ValueError("q_col must be 2-D")
        rows_out, layout = qc.shape[1], MXFP8_CANONICAL
        if tuple(qc.shape) != (cols, rows_out) or tuple(sc.shape) != (cols, rows_out // 32):
            raise ValueError("q_col/s_col must be [cols, rows_out] / [cols, rows_out/32]")
    if rows % 32 or cols % 32 or rows_out % 32:
        raise ValueError("rows, cols and rows_out must be multiples of 32")
    if row_out is not None:
        if not isinstance(row_out, PackedWeight) or (row_out.batch, row_out.N, row_out.K) != (1, rows, cols):
            raise ValueError("row_out must be PackedWeight(batch 1, N = %d, K = %d)" % (rows, cols))
        outs.append((row_out, (rows, cols), "row_out"))
    for t, (n, k), name in outs:
        _need(t.q, torch.uint8, name + ".q")
        _need(t.s, torch.uint8, name + ".s")
        if t.q.numel() < packed_bytes(1, n, k, 0) or t.s.numel() < packed_bytes(1, n, k, 1):
            raise ValueError("%s buffers too small" % name)
    _check(lib().mxfp8_quantize_dual_grouped_packed(
        _ptr(x), rows, cols, _ptr(row_out.q) if row_out is not None else None,
        _ptr(row_out.s) if row_out is not None else None, _ptr(qc), _ptr(sc), layout, _ptr(src_offsets),
        _ptr(dst_offsets), G, rows_out, _stream(x.device)), "mxfp8_quantize_dual_grouped_packed")


def quantize_dual_grouped(x: torch.Tensor, src_offsets: torch.Tensor, dst_offsets: torch.Tensor, rows_out: int,
                          row_grid: bool = True):
    """-> (q_row, s_row, q_col, s_col) (the first two None unless row_grid)."""
    rows, cols = x.shape
    q_col = torch.empty((cols, rows_out), dtype=torch.uint8, device=x.device)
    s_col = torch.empty((cols, rows_out // 32), dtype=torch.uint8, device=x.device)
    q_row = s_row = None
    if row_grid:
        q_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        s_row = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    quantize_dual_grouped_into(x, src_offsets, dst_offsets, q_col, s_col, q_row, s_row)
    return q_row, s_row, q_col, s_col


def dequantize(q: torch.Tensor, s: torch.Tensor, rows: int, cols: int, axis: int = 1,
               dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    _need(q, torch.uint8, "q")
    _need(s, torch.uint8, "scales")
    code = _out_code(dtype)
    if q.numel() != rows * cols:
        raise ValueError("q has %d elements, expected %d" % (q.numel(), rows * cols))
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=q.device)
    else:
        _need(out, dtype, "out")
    _check(lib().mxfp8_dequantize(_ptr(q), _ptr(s), rows, cols, axis, _ptr(out), code,
                                  _stream(q.device)), "mxfp8_dequantize")
    return out


# ------------------------------------------------------------------ repack

def packed_bytes(batch: int, rows: int, cols: int, which: int) -> int:
    return int(lib().mxfp8_packed_bytes(batch, rows, cols, which))


@dataclass
class PackedWeight:
    """Weights [batch][N][K] in the GEMM's kernel layout (mxfp8_repack)."""
    q: torch.Tensor
    s: torch.Tensor
    batch: int
    N: int
    K: int


def repack_(q: torch.Tensor, s: torch.Tensor, w: PackedWeight) -> PackedWeight:
    """Rebuild the kernel layout in place into w's storage (pointers stay valid)."""
    _need(q, torch.uint8, "q")
    _need(s, torch.uint8, "scales")
    _need(w.q, torch.uint8, "q_packed")
    _need(w.s, torch.uint8, "scales_packed")
    if q.numel() != w.batch * w.N * w.K or s.numel() != w.batch * w.N * (w.K // 32):
        raise ValueError("canonical q/scales do not match the packed weight's shape")
    if w.q.numel() < packed_bytes(w.batch, w.N, w.K, 0) or w.s.numel() < packed_bytes(w.batch, w.N, w.K, 1):
        raise ValueError("packed buffers too small")
    _check(lib().mxfp8_repack(_ptr(q), _ptr(s), w.batch, w.N, w.K, _ptr(w.q), _ptr(w.s),
                              _stream(q.device)), "mxfp8_repack")
    return w


def repack(q: torch.Tensor, s: torch.Tensor) -> PackedWeight:
    """Canonical q[(batch,) N, K], s[(batch,) N, K/32] -> PackedWeight."""
    if q.dim() == 2:
        batch, (N, K) = 1, q.shape
    elif q.dim() == 3:
        batch, N, K = q.shape
    else:
        raise ValueError("q must be [N, K] or [batch, N, K]")
    nq, ns = packed_bytes(batch, N, K, 0), packed_bytes(batch, N, K, 1)
    if nq == 0:
        raise ValueError("invalid weight shape for packing")
    w = PackedWeight(torch.empty(nq, dtype=torch.uint8, device=q.device),
                     torch.empty(ns, dtype=torch.uint8, device=q.device), batch, N, K)
    return repack_(q, s, w)


def quantize_packed_(w_bf16: torch.Tensor, out: PackedWeight, q: torch.Tensor | None = None,
                     s: torch.Tensor | None = None) -> PackedWeight:
    """Quantize weights [(batch,) N, K] along K straight into out's packed
    storage (in place), and into the canonical (q, s) as well if given."""
    _need(w_bf16, torch.bfloat16, "w")
    _need(out.q, torch.uint8, "q_packed")
    _need(out.s, torch.uint8, "scales_packed")
    if w_bf16.numel() != out.batch * out.N * out.K:
        raise ValueError("weights do not match the packed weight's shape")
    if out.q.numel() < packed_bytes(out.batch, out.N, out.K, 0) or \
            out.s.numel() < packed_bytes(out.batch, out.N, out.K, 1):
        raise ValueError("packed buffers too small")
    if (q is None) != (s is None):
        raise ValueError("give both canonical q and scales, or neither")
    if q is not None:
        _need(q, torch.uint8, "q")
        _need(s, torch.uint8, "scales")
        if q.numel() != w_bf16.numel() or s.numel() != w_bf16.numel() // 32:
            raise ValueError("canonical q/scales have the wrong size")
    _check(lib().mxfp8_quantize_packed(_ptr(w_bf16), out.batch, out.N, out.K,
                                       _ptr(q) if q is not None else None,
                                       _ptr(s) if s is not None else None,
                                       _ptr(out.q), _ptr(out.s), _stream(w_bf16.device)),
           "mxfp8_quantize_packed")
    return out


def quantize_packed_axis0_(x_bf16: torch.Tensor, out: PackedWeight) -> PackedWeight:
    """x [(batch,) rows, cols] quantized along rows (axis 0) straight into the
    packed layout of its transposed grid: out is PackedWeight(batch, N=cols,
    K=rows), equal to repack(quantize_batched(x, 0))."""
    _need(x_bf16, torch.bfloat16, "x")
    _need(out.q, torch.uint8, "q_packed")
    _need(out.s, torch.uint8, "scales_packed")
    if x_bf16.dim() == 2:
        batch, (rows, cols) = 1, x_bf16.shape
    elif x_bf16.dim() == 3:
        batch, rows, cols = x_bf16.shape
    else:
        raise ValueError("x must be [rows, cols] or [batch, rows, cols]")
    if (out.batch, out.N, out.K) != (batch, cols, rows):
        raise ValueError("packed weight must be (batch, N=cols, K=rows) = %s" % ((batch, cols, rows),))
    if out.q.numel() < packed_bytes(batch, cols, rows, 0) or out.s.numel() < packed_bytes(batch, cols, rows, 1):
        raise ValueError("packed buffers too small")
    _check(lib().mxfp8_quantize_packed_axis0(_ptr(x_bf16), batch, rows, cols, _ptr(out.q), _ptr(out.s),
                                             _stream(x_bf16.device)), "mxfp8_quantize_packed_axis0")
    return out


def quantize_many_(items) -> None:
    """quantize_into(x, 1, q, s) over a list of (x_bf16, q, s) in launches of
    up to QUANT_JOBS_MAX tensors (mxfp8_quantize_many), on the current stream
    of the first tensor's device."""
    items = list(items)
    jobs = []
    for x, q, s in items:
        _need(x, torch.bfloat16, "x")
        _need(q, torch.uint8, "q")
        _need(s, torch.uint8, "scales")
        if x.dim() != 2:
            raise ValueError("x must be 2-D [rows, cols]")
        rows, cols = x.shape
        if tuple(q.shape) != (rows, cols) or tuple(s.shape) != (rows, cols // 32):
            raise ValueError("q/scales shapes %s/%s, expected %s/%s" % (tuple(q.shape), tuple(s.shape),
                                                                      (rows, cols), (rows, cols // 32)))
        if x.device != items[0][0].device:
            raise ValueError("all tensors must be on one device")
        jobs.append(QuantJob(x.data_ptr(), rows, cols, q.data_ptr(), s.data_ptr()))
    if not jobs:
        return
    stream = _stream(items[0][0].device)
    for i in range(0, len(jobs), QUANT_JOBS_MAX):
        chunk = jobs[i:i + QUANT_JOBS_MAX]
        arr = (QuantJob * len(chunk))(*chunk)
        _check(lib().mxfp8_quantize_many(arr, len(chunk), stream), "mxfp8_quantize_many")


def quantize_many_layouts_(items) -> None:
    """Axis-1 quantize of a list of (x_bf16 [rows, cols], target) in one launch
    (mxfp8_quantize_many_layouts, up to QUANT_JOBS_MAX entries): target is a
    canonical (q, s) pair, or a PackedWeight (batch 1, N = rows, K = cols)
    that receives the packed layout (the operand layout of gemm_packed)."""
    items = list(items)
    if not items or len(items) > QUANT_JOBS_MAX:
        raise ValueError("1 to %d entries" % QUANT_JOBS_MAX)
    jobs = []
    for x, target in items:
        _need(x, torch.bfloat16, "x")
        if x.dim() != 2:
            raise ValueError("x must be 2-D [rows, cols]")
        rows, cols = x.shape
        if x.device != items[0][0].device:
            raise ValueError("all tensors must be on one device")
        if isinstance(target, PackedWeight):
            _need(target.q, torch.uint8, "q_packed")
            _need(target.s, torch.uint8, "scales_packed")
            if (target.batch, target.N, target.K) != (1, rows, cols):
                raise ValueError("packed target must be PackedWeight(batch 1, N = rows, K = cols)")
            if target.q.numel() < packed_bytes(1, rows, cols, 0) or target.s.numel() < packed_bytes(1, rows, cols, 1):
                raise ValueError("packed buffers too small")
            jobs.append(QuantLayoutJob(x.data_ptr(), rows, cols, MXFP8_PACKED, target.q.data_ptr(),
                                       target.s.data_ptr()))
        else:
            q, s = target
            _need(q, torch.uint8, "q")
            _need(s, torch.uint8, "scales")
            if tuple(q.shape) != (rows, cols) or tuple(s.shape) != (rows, cols // 32):
                raise ValueError("q/scales shapes do not match x")
            jobs.append(QuantLayoutJob(x.data_ptr(), rows, cols, MXFP8_CANONICAL, q.data_ptr(), s.data_ptr()))
    arr = (QuantLayoutJob * len(jobs))(*jobs)
    _check(lib().mxfp8_quantize_many_layouts(arr, len(jobs), _stream(items[0][0].device)),
           "mxfp8_quantize_many_layouts")


def quantize_packed_many_(items) -> None:
    """quantize_packed_ over a list of (w_bf16, PackedWeight or None, q or
    None, s or None) in launches of up to PACKED_JOBS_MAX weights
    (mxfp8_quantize_packed_many), all on the current stream of the first
    weight's device.  An entry without a PackedWeight writes only its
    canonical grid (q and s given)."""
    items = list(items)
    jobs = []
    for w_bf16, out, q, s in items:
        _need(w_bf16, torch.bfloat16, "w")
        if out is None:
            if q is None:
                raise ValueError("an entry needs the packed layout, the canonical grid, or both")
            shape = tuple(w_bf16.shape)
            if len(shape) not in (2, 3):
                raise ValueError("weights must be [N, K] or [batch, N, K]")
            batch, (N, K) = (1, shape) if len(shape) == 2 else (shape[0], shape[1:])
        else:
            _need(out.q, torch.uint8, "q_packed")
            _need(out.s, torch.uint8, "scales_packed")
            batch, N, K = out.batch, out.N, out.K
            if w_bf16.numel() != batch * N * K:
                raise ValueError("weights do not match the packed weight's shape")
            if out.q.numel() < packed_bytes(batch, N, K, 0) or out.s.numel() < packed_bytes(batch, N, K, 1):
                raise ValueError("packed buffers too small")
        if (q is None) != (s is None):
            raise ValueError("give both canonical q and scales, or neither")
        if q is not None:
            _need(q, torch.uint8, "q")
            _need(s, torch.uint8, "scales")
            if q.numel() != w_bf16.numel() or s.numel() != w_bf16.numel() // 32:
                raise ValueError("canonical q/scales have the wrong size")
        if w_bf16.device != items[0][0].device:
            raise ValueError("all weights must be on one device")
        jobs.append(PackedJob(w_bf16.data_ptr(), batch, N, K,
                              q.data_ptr() if q is not None else None,
                              s.data_ptr() if s is not None else None,
                              out.q.data_ptr() if out is not None else None,
                              out.s.data_ptr() if out is not None else None))
    if not jobs:
        return
    stream = _stream(items[0][0].device)
    for i in range(0, len(jobs), PACKED_JOBS_MAX):
        chunk = jobs[i:i + PACKED_JOBS_MAX]
        arr = (PackedJob * len(chunk))(*chunk)
        _check(lib().mxfp8_quantize_packed_many(arr, len(chunk), stream), "mxfp8_quantize_packed_many")


def quantize_packed(w_bf16: torch.Tensor, canonical: bool = True):
    """Weights [(batch,) N, K] -> (PackedWeight, q, s) in one pass; q and s
    (the canonical grid) are None when canonical is False."""
    if w_bf16.dim() == 2:
        batch, (N, K) = 1, w_bf16.shape
    elif w_bf16.dim() == 3:
        batch, N, K = w_bf16.shape
    else:
        raise ValueError("weights must be [N, K] or [batch, N, K]")
    nq, ns = packed_bytes(batch, N, K, 0), packed_bytes(batch, N, K, 1)
    if nq == 0:
        raise ValueError("invalid weight shape for packing")
    out = PackedWeight(torch.empty(nq, dtype=torch.uint8, device=w_bf16.device),
                       torch.empty(ns, dtype=torch.uint8, device=w_bf16.device), batch, N, K)
    q = s = None
    if canonical:
        q = torch.empty(tuple(w_bf16.shape), dtype=torch.uint8, device=w_bf16.device)
        s = torch.empty(tuple(w_bf16.shape[:-1]) + (K // 32,), dtype=torch.uint8, device=w_bf16.device)
    quantize_packed_(w_bf16, out, q, s)
    return out, q, s


# ------------------------------------------------------------------ GEMMs

def gemm_splitk_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes gemm_splitk uses for this shape on the current device (0: no split)."""
    return int(lib().mxfp8_gemm_splitk_workspace_bytes(M, N, K))


def gemm(a_q: torch.Tensor, a_s: torch.Tensor, b, out_dtype=torch.bfloat16,
         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         split_k: bool = False, accurate: bool = False) -> torch.Tensor:
    """C[M, N] = A[M, K] B[N, K]^T.  ``b`` is a PackedWeight (batch 1) or a
    canonical (b_q[N, K], b_s[N, K/32]) pair.  With split_k (or a workspace
    given) the call is mxfp8_gemm_splitk: K split over workgroups when the
    shape has few output tiles, partials in ``workspace`` (a uint8 device
    tensor; allocated here, through torch, when not given).  With accurate
    the call is mxfp8_gemm_accurate (exact products, fp32-accurate sums)."""
    _need(a_q, torch.uint8, "a_q")
    _need(a_s, torch.uint8, "a_s")
    M, K = a_q.shape
    if isinstance(b, PackedWeight):
        if b.batch != 1 or b.K != K:
            raise ValueError("packed B must be a single [N, K] matrix with K = %d" % K)
        b_q, b_s, N, layout = b.q, b.s, b.N, MXFP8_PACKED
    else:
        b_q, b_s = b
        _need(b_q, torch.uint8, "b_q")
        _need(b_s, torch.uint8, "b_s")
        N = b_q.shape[0]
        if b_q.shape[1] != K or tuple(b_s.shape) != (N, K // 32):
            raise ValueError("canonical B shapes do not match K = %d" % K)
        layout = MXFP8_CANONICAL
    if tuple(a_s.shape) != (M, K // 32):
        raise ValueError("a_s must be [M, K/32]")
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    else:
        _need(out, out_dtype, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    if accurate:
        if split_k or workspace is not None:
            raise ValueError("accurate and split_k are separate calls")
        _check(lib().mxfp8_gemm_accurate(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), layout, M, N, K,
                                         _ptr(out), code, _stream(a_q.device)), "mxfp8_gemm_accurate")
        return out
    if split_k or workspace is not None:
        need = gemm_splitk_workspace_bytes(M, N, K)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=a_q.device)
        if workspace is not None:
            _need(workspace, torch.uint8, "workspace")
        _check(lib().mxfp8_gemm_splitk(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), layout, M, N, K, _ptr(out),
                                       code, _ptr(workspace) if workspace is not None else None,
                                       workspace.numel() if workspace is not None else 0, _stream(a_q.device)),
               "mxfp8_gemm_splitk")
        return out
    _check(lib().mxfp8_gemm(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), layout, M, N, K,
                            _ptr(out), code, _stream(a_q.device)), "mxfp8_gemm")
    return out


def gemm_packed(a: PackedWeight, b: PackedWeight, out_dtype=torch.bfloat16,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                split_k: bool = False) -> torch.Tensor:
    """C[M, N] = A[M, K] B[N, K]^T with both operands in the packed layout
    (mxfp8_gemm_packed): A from quantize_packed / repack of [M, K] (a.N = M),
    B a packed weight.  K % 128 == 0.  With split_k (or a workspace given)
    the call is mxfp8_gemm_packed_splitk, its workspace sized as
    gemm_splitk's (allocated here, through torch, when not given)."""
    for name, w in (("a", a), ("b", b)):
        if not isinstance(w, PackedWeight) or w.batch != 1:
            raise ValueError("%s must be a single packed [rows, K] matrix" % name)
        _need(w.q, torch.uint8, name + ".q")
        _need(w.s, torch.uint8, name + ".s")
    if a.K != b.K:
        raise ValueError("A and B must share K")
    M, N, K = a.N, b.N, a.K
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.q.device)
    else:
        _need(out, out_dtype, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    if split_k or workspace is not None:
        need = gemm_splitk_workspace_bytes(M, N, K)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=a.q.device)
        if workspace is not None:
            _need(workspace, torch.uint8, "workspace")
        _check(lib().mxfp8_gemm_packed_splitk(_ptr(a.q), _ptr(a.s), _ptr(b.q), _ptr(b.s), M, N, K, _ptr(out), code,
                                              _ptr(workspace) if workspace is not None else None,
                                              workspace.numel() if workspace is not None else 0,
                                              _stream(a.q.device)), "mxfp8_gemm_packed_splitk")
        return out
    _check(lib().mxfp8_gemm_packed(_ptr(a.q), _ptr(a.s), _ptr(b.q), _ptr(b.s), M, N, K, _ptr(out), code,
                                   _stream(a.q.device)), "mxfp8_gemm_packed")
    return out


def grouped_gemm(a_q: torch.Tensor, a_s: torch.Tensor, w: PackedWeight, offsets: torch.Tensor,
                 out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-expert C[o_g:o_g+1] = A[o_g:o_g+1] B_g^T with device int32 offsets [G+1]."""
    _need(a_q, torch.uint8, "a_q")
    _need(a_s, torch.uint8, "a_s")
    _need(offsets, torch.int32, "offsets")
    M_total, K = a_q.shape
    if w.K != K:
        raise ValueError("K mismatch")
    G = w.batch
    if offsets.numel() != G + 1:
        raise ValueError("offsets must have G + 1 = %d entries" % (G + 1))
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((M_total, w.N), dtype=out_dtype, device=a_q.device)
    else:
        _need(out, out_dtype, "out")
        if tuple(out.shape) != (M_total, w.N):
            raise ValueError("out must be [M_total, N]")
    if tuple(a_s.shape) != (M_total, K // 32):
        raise ValueError("a_s must be [M_total, K/32]")
    _check(lib().mxfp8_grouped_gemm(_ptr(a_q), _ptr(a_s), _ptr(w.q), _ptr(w.s), _ptr(offsets), G,
                                    M_total, w.N, K, _ptr(out), code, _stream(a_q.device)),
           "mxfp8_grouped_gemm")
    return out


def grouped_gemm_packed(a: PackedWeight, w: PackedWeight, offsets: torch.Tensor,
                        out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """grouped_gemm with A in the packed layout (mxfp8_grouped_gemm_packed):
    ``a`` is the packed layout of the [M_total, K] rows (batch 1, a.N =
    M_total), e.g. from quantize_many_layouts_; K % 128 == 0."""
    for name, t in (("a", a), ("w", w)):
        if not isinstance(t, PackedWeight):
            raise ValueError("%s must be a PackedWeight" % name)
        _need(t.q, torch.uint8, name + ".q")
        _need(t.s, torch.uint8, name + ".s")
    if a.batch != 1:
        raise ValueError("a must be a single packed [M_total, K] matrix")
    _need(offsets, torch.int32, "offsets")
    M_total, K = a.N, a.K
    if w.K != K:
        raise ValueError("K mismatch")
    G = w.batch
    if offsets.numel() != G + 1:
        raise ValueError("offsets must have G + 1 = %d entries" % (G + 1))
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((M_total, w.N), dtype=out_dtype, device=a.q.device)
    else:
        _need(out, out_dtype, "out")
        if tuple(out.shape) != (M_total, w.N):
            raise ValueError("out must be [M_total, N]")
    _check(lib().mxfp8_grouped_gemm_packed(_ptr(a.q), _ptr(a.s), _ptr(w.q), _ptr(w.s), _ptr(offsets), G,
                                           M_total, w.N, K, _ptr(out), code, _stream(a.q.device)),
           "mxfp8_grouped_gemm_packed")
    return out


def grouped_gemm_wgrad(a_q: torch.Tensor, a_s: torch.Tensor, b_q: torch.Tensor, b_s: torch.Tensor,
                       offsets: torch.Tensor, out_dtype=torch.float32,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """C[g] = A[:, o_g:o_g+1] B[:, o_g:o_g+1]^T for A [M, T], B [N, T] quantized
    along tokens (axis-0 outputs) and device int32 token offsets [G+1]."""
    for t, n in ((a_q, "a_q"), (a_s, "a_s"), (b_q, "b_q"), (b_s, "b_s")):
        _need(t, torch.uint8, n)
    _need(offsets, torch.int32, "offsets")
    M, T = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != T or tuple(a_s.shape) != (M, T // 32) or tuple(b_s.shape) != (N, T // 32):
        raise ValueError("A [M, T] and B [N, T] with scales [., T/32] expected")
    G = offsets.numel() - 1
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((G, M, N), dtype=out_dtype, device=a_q.device)
    else:
        _need(out, out_dtype, "out")
        if tuple(out.shape) != (G, M, N):
            raise ValueError("out must be [G, M, N]")
    _check(lib().mxfp8_grouped_gemm_wgrad(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(offsets), G,
                                          T, M, N, _ptr(out), code, _stream(a_q.device)),
           "mxfp8_grouped_gemm_wgrad")
    return out


def grouped_gemm_wgrad_packed(a: "PackedWeight", b: "PackedWeight", offsets: torch.Tensor, out_dtype=torch.float32,
                              out: torch.Tensor | None = None) -> torch.Tensor:
    """mxfp8_grouped_gemm_wgrad_packed: C[g] = A[:, K_g] B[:, K_g]^T with A =
    PackedWeight(batch 1, N = M, K = T) and B = PackedWeight(batch 1, N, T)
    (the regrouped token-blocked grids in the packed layout) and device int32
    token offsets [G+1] (multiples of 128)."""
    for name, w in (("a", a), ("b", b)):
        if not isinstance(w, PackedWeight) or w.batch != 1:
            raise ValueError("%s must be a single packed [rows, T] matrix" % name)
        _need(w.q, torch.uint8, name + ".q")
        _need(w.s, torch.uint8, name + ".s")
    _need(offsets, torch.int32, "offsets")
    if a.K != b.K:
        raise ValueError("A and B must share the token axis")
    M, N, T = a.N, b.N, a.K
    G = offsets.numel() - 1
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((G, M, N), dtype=out_dtype, device=a.q.device)
    else:
        _need(out, out_dtype, "out")
        if tuple(out.shape) != (G, M, N):
            raise ValueError("out must be [G, M, N]")
    _check(lib().mxfp8_grouped_gemm_wgrad_packed(_ptr(a.q), _ptr(a.s), _ptr(b.q), _ptr(b.s), _ptr(offsets), G, T, M,
                                                 N, _ptr(out), code, _stream(a.q.device)),
           "mxfp8_grouped_gemm_wgrad_packed")
    return out


# ------------------------------------------------------------------ self-check

SELFCHECK_TOLERANCE = 0.25


def selfcheck_rel_err(w_q: torch.Tensor, w_s: torch.Tensor, packed: PackedWeight, index: int = 0,
                      probe_rows: int = 128, seed: int = 0, x: torch.Tensor | None = None):
    """Relative Frobenius error of matrix `index` of `packed` served by the
    MXFP8 GEMM on a random N(0,1) probe against an fp32 GEMM on the
    dequantized canonical grid (w_q [N, K], w_s [N, K/32] of that matrix).
    Returns (rel_err, sum_sq_err, sum_sq_ref); rel_err is NaN if an output is
    not finite.  Synchronizes the current stream to read the verdict."""
    N, K = packed.N, packed.K
    _need(w_q, torch.uint8, "w_q")
    _need(w_s, torch.uint8, "w_s")
    if w_q.numel() != N * K or w_s.numel() != N * (K // 32):
        raise ValueError("w_q/w_s must be one [N, K] canonical matrix")
    if not 0 <= index < packed.batch:
        raise ValueError("matrix index out of range")
    dev = w_q.device
    if x is None:
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        x = torch.randn((probe_rows, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    _need(x, torch.bfloat16, "x")
    M = x.shape[0]
    nbytes = int(lib().mxfp8_selfcheck_workspace_bytes(M, N, K))
    if nbytes == 0:
        raise ValueError("unsupported self-check size")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    res = torch.empty(3, dtype=torch.float64, device=dev)
    oq = index * packed_bytes(1, N, K, 0)
    os_ = index * packed_bytes(1, N, K, 1)
    _check(lib().mxfp8_selfcheck(_ptr(x), M, N, K, _ptr(w_q), _ptr(w_s),
                                 ctypes.c_void_p(packed.q.data_ptr() + oq),
                                 ctypes.c_void_p(packed.s.data_ptr() + os_),
                                 _ptr(ws), _ptr(res), _stream(dev)), "mxfp8_selfcheck")
    torch.cuda.current_stream(dev).synchronize()
    r = res.cpu().tolist()
    return r[0], r[1], r[2]
