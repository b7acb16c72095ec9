"""GPU parity of the fused quantizers against the oracle, bit for bit.

mxfp8_quantize_dual must equal the oracle's quantize along both axes, and
mxfp8_quantize_packed must equal the oracle's packing of its axis-1 quantize
(plus the canonical grid when requested) -- the definitions both calls state
in include/mxfp8.h.  Shapes span several 128x128 (dual) or 256x128 (packed)
tiles with ragged edges, the full learner and weight-sync shapes, and the
special values (zero, subnormal, NaN and Inf blocks).
"""
import numpy as np
import pytest

import workloads as wl
from conftest import to_dev, to_host

pytestmark = pytest.mark.gpu


def _say(*a):
    print("fused case:", *a, flush=True)


def _specials(x, rng):
    """Plant zero, subnormal, NaN, Inf and large-magnitude blocks into a BF16 array."""
    x = x.copy()
    flat = x.reshape(-1)
    nblk = flat.size // 32
    picks = rng.choice(nblk, size=min(nblk, 12), replace=False)
    kinds = [0x0000, 0x0001, 0x7FC0, 0x7F80, 0xFF80, 0x7F7F, 0x8000, 0x0080]
    for i, b in enumerate(picks):
        kind = kinds[i % len(kinds)]
        lo = b * 32
        if kind in (0x0000, 0x8000):
            flat[lo:lo + 32] = kind                              # all-zero block (signed)
        elif kind in (0x0001, 0x0080):
            flat[lo:lo + 32] = kind + rng.integers(0, 64, 32)   # subnormals / smallest normals
        else:
            flat[lo + int(rng.integers(0, 32))] = kind           # one NaN / Inf / max in the block
    return x


@pytest.mark.parametrize("rows,cols", [(32, 32), (64, 96), (160, 224), (256, 384), (96, 4160),
                                       (4096, 4096)])
def test_quantize_dual_matches_both_axes(mx, oracle_mod, rows, cols):
    _say("dual", rows, cols)
    rng = np.random.default_rng(rows * 7 + cols)
    x = wl.normal_bf16(rng, (rows, cols), outlier_frac=0.01)
    if rows * cols <= 1 << 20:
        x = _specials(x, rng)
    q1, s1, q0, s0 = mx.quantize_dual(to_dev(x))
    rq1, rs1 = oracle_mod.quantize(x, 1)
    rq0, rs0 = oracle_mod.quantize(x, 0)
    assert np.array_equal(to_host(q1), rq1) and np.array_equal(to_host(s1), rs1)
    assert np.array_equal(to_host(q0), rq0) and np.array_equal(to_host(s0), rs0)


def test_quantize_dual_mlp_gradient_full_size(mx, oracle_mod):
    """dY_gu of the MLP micro-batch (8192 x 24576), the largest learner tensor."""
    _say("dual mlp dY_gu")
    rng = np.random.default_rng(11)
    x = wl.normal_bf16(rng, (8192, 24576), std=2.0 ** -10)
    q1, s1, q0, s0 = mx.quantize_dual(to_dev(x))
    rq1, rs1 = oracle_mod.quantize(x, 1)
    assert np.array_equal(to_host(q1), rq1) and np.array_equal(to_host(s1), rs1)
    del rq1, rs1
    rq0, rs0 = oracle_mod.quantize(x, 0)
    assert np.array_equal(to_host(q0), rq0) and np.array_equal(to_host(s0), rs0)


@pytest.mark.parametrize("batch,N,K", [(1, 256, 128), (1, 300, 320), (3, 17, 96), (2, 512, 768),
                                       (5, 1000, 1056), (1, 6144, 4096), (16, 1536, 2048)])
@pytest.mark.parametrize("canonical", [False, True])
def test_quantize_packed_matches_quantize_then_pack(mx, oracle_mod, batch, N, K, canonical):
    _say("packed", batch, N, K, canonical)
    rng = np.random.default_rng(batch * 1000 + N + K)
    w = wl.normal_bf16(rng, (batch * N, K), std=0.02)
    if batch * N * K <= 1 << 21:
        w = _specials(w, rng)
    pw, q, s = mx.quantize_packed(to_dev(w.reshape(batch, N, K)), canonical=canonical)
    rq, rs = oracle_mod.quantize(w, 1)
    qp_ref, sp_ref = oracle_mod.pack(rq.reshape(batch, N, K), rs.reshape(batch, N, K // 32), batch, N, K)
    assert np.array_equal(to_host(pw.q), qp_ref)
    assert np.array_equal(to_host(pw.s), sp_ref)
    if canonical:
        assert np.array_equal(to_host(q).reshape(batch * N, K), rq)
        assert np.array_equal(to_host(s).reshape(batch * N, K // 32), rs)
    else:
        assert q is None and s is None


def test_quantize_packed_feeds_gemm_like_repack(mx, oracle_mod):
    """The packed bytes are the repack bytes, so the GEMM result is identical."""
    import torch
    _say("packed gemm")
    rng = np.random.default_rng(5)
    M, N, K = 96, 300, 512
    w = wl.normal_bf16(rng, (N, K), std=0.02)
    x = wl.normal_bf16(rng, (M, K))
    xq, xs = mx.quantize(to_dev(x), 1)
    pw, q, s = mx.quantize_packed(to_dev(w))
    ref = mx.repack(q, s)
    y1 = mx.gemm(xq, xs, pw, torch.float32)
    y2 = mx.gemm(xq, xs, ref, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(y1), to_host(y2))


def _packed_out(mx, batch, N, K, canonical, dev):
    """Output buffers of one weight, filled with 0xEE so an unwritten byte shows."""
    import torch
    pw = mx.PackedWeight(torch.full((mx.packed_bytes(batch, N, K, 0),), 0xEE, dtype=torch.uint8, device=dev),
                         torch.full((mx.packed_bytes(batch, N, K, 1),), 0xEE, dtype=torch.uint8, device=dev),
                         batch, N, K)
    q = s = None
    if canonical:
        q = torch.full((batch, N, K), 0xEE, dtype=torch.uint8, device=dev)
        s = torch.full((batch, N, K // 32), 0xEE, dtype=torch.uint8, device=dev)
    return pw, q, s


def test_quantize_packed_many_matches_oracle(mx, oracle_mod):
    """34 ragged weights (two launches: 32 + 2), canonical grid on every other
    one and only the canonical grid on every sixth: each equals the oracle's
    quantize + pack."""
    import torch
    shapes = [(1, 256, 128), (1, 300, 320), (3, 17, 96), (2, 512, 768), (1, 40, 4160), (1, 513, 96),
              (1, 1, 32), (2, 257, 160), (1, 1024, 256), (1, 96, 1056), (4, 33, 64), (1, 768, 512),
              (1, 255, 384), (1, 64, 2048), (2, 130, 224), (1, 2048, 128), (1, 7, 4096), (3, 300, 96)]
    shapes = shapes + shapes[:16]
    _say("packed many", len(shapes))
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(77)
    items, refs = [], []
    for i, (batch, N, K) in enumerate(shapes):
        w = wl.normal_bf16(rng, (batch * N, K), std=0.02 * (1 + i))
        w = _specials(w, rng)
        pw, q, s = _packed_out(mx, batch, N, K, i % 2 == 0, dev)
        if i % 6 == 4:
            pw = None
        items.append((to_dev(w.reshape(batch, N, K)), pw, q, s))
        refs.append(w)
    mx.quantize_packed_many_(items)
    torch.cuda.synchronize()
    for (batch, N, K), w, (_, pw, q, s) in zip(shapes, refs, items):
        rq, rs = oracle_mod.quantize(w, 1)
        qp_ref, sp_ref = oracle_mod.pack(rq.reshape(batch, N, K), rs.reshape(batch, N, K // 32), batch, N, K)
        if pw is not None:
            assert np.array_equal(to_host(pw.q), qp_ref), (batch, N, K)
            assert np.array_equal(to_host(pw.s), sp_ref), (batch, N, K)
        if q is not None:
            assert np.array_equal(to_host(q).reshape(batch * N, K), rq), (batch, N, K)
            assert np.array_equal(to_host(s).reshape(batch * N, K // 32), rs), (batch, N, K)


def test_quantize_packed_many_sync_layer(mx, oracle_mod):
    """One Qwen3-8B layer's four linears in one launch (its input is above the
    nontemporal threshold) equal the per-weight calls byte for byte, and the
    qkv and down weights equal the oracle."""
    import torch
    _say("packed many, qwen3-8b layer")
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(78)
    items, singles, hosts = [], [], {}
    for name, N, K in wl.sync_layer_shapes():
        w = wl.normal_bf16(rng, (N, K), std=0.02)
        wd = to_dev(w)
        if name in ("qkv", "down"):
            hosts[name] = w
        items.append((wd,) + _packed_out(mx, 1, N, K, True, dev))
        singles.append(mx.quantize_packed(wd, canonical=True))
    mx.quantize_packed_many_(items)
    torch.cuda.synchronize()
    for (name, N, K), (_, pw, q, s), (pw1, q1, s1) in zip(wl.sync_layer_shapes(), items, singles):
        assert torch.equal(pw.q, pw1.q) and torch.equal(pw.s, pw1.s), name
        assert torch.equal(q.view(N, K), q1) and torch.equal(s.view(N, K // 32), s1), name
        if name in hosts:
            rq, rs = oracle_mod.quantize(hosts[name], 1)
            assert np.array_equal(to_host(q).reshape(N, K), rq), name
            assert np.array_equal(to_host(s).reshape(N, K // 32), rs), name
            qp_ref, sp_ref = oracle_mod.pack(rq.reshape(1, N, K), rs.reshape(1, N, K // 32), 1, N, K)
            assert np.array_equal(to_host(pw.q), qp_ref), name
            assert np.array_equal(to_host(pw.s), sp_ref), name


@pytest.mark.parametrize("batch,rows,cols", [(1, 128, 256), (1, 96, 40), (3, 64, 296), (2, 320, 520),
                                             (1, 32, 8), (4, 1536, 2048), (2, 2048, 768)])
def test_quantize_packed_axis0_matches_quantize_then_pack(mx, oracle_mod, batch, rows, cols):
    """mxfp8_quantize_packed_axis0 equals the oracle's axis-0 quantize of each
    matrix packed as the transposed grid (N = cols, K = rows), padding
    included; half-panels beyond cols and k-steps beyond rows are covered."""
    import torch
    _say("packed axis0", batch, rows, cols)
    rng = np.random.default_rng(batch * 7 + rows * 3 + cols)
    x = wl.normal_bf16(rng, (batch * rows, cols), std=0.02)
    if batch * rows * cols <= 1 << 21:
        x = _specials(x, rng)
    dev = torch.device("cuda:0")
    pw = _packed_out(mx, batch, cols, rows, False, dev)[0]
    mx.quantize_packed_axis0_(to_dev(x.reshape(batch, rows, cols)), pw)
    torch.cuda.synchronize()
    q0 = np.empty((batch, cols, rows), np.uint8)
    s0 = np.empty((batch, cols, rows // 32), np.uint8)
    for b in range(batch):
        q0[b], s0[b] = oracle_mod.quantize(np.ascontiguousarray(x[b * rows:(b + 1) * rows]), 0)
    qp_ref, sp_ref = oracle_mod.pack(q0, s0, batch, cols, rows)
    assert np.array_equal(to_host(pw.q), qp_ref)
    assert np.array_equal(to_host(pw.s), sp_ref)


def test_quantize_packed_axis0_mlp_weight_full_size(mx):
    """The MLP gate_up weight [24576 x 4096] (input above the nontemporal
    threshold): equal to quantize(axis 0) + repack on the device, byte for byte."""
    import torch
    _say("packed axis0 mlp W_gu")
    dev = torch.device("cuda:0")
    W = wl.torch_normal_bf16((24576, 4096), 0.02, seed=5, device=dev)
    pw = _packed_out(mx, 1, 4096, 24576, False, dev)[0]
    mx.quantize_packed_axis0_(W, pw)
    q0, s0 = mx.quantize(W, 0)
    ref = mx.repack(q0, s0)
    torch.cuda.synchronize()
    assert torch.equal(pw.q, ref.q) and torch.equal(pw.s, ref.s)


@pytest.mark.parametrize("rows,cols", [(32, 32), (96, 160), (288, 416), (512, 384), (64, 4160), (8192, 4096)])
def test_quantize_dual_packed_matches_pack_of_both_axes(mx, oracle_mod, rows, cols):
    """mxfp8_quantize_dual_packed equals the oracle's packing of its quantize
    along each axis (padding rows, blocks and half panels included), on
    special values; the MLP activation shape (8192 x 4096) against
    mxfp8_quantize_dual + mxfp8_repack on the device."""
    import torch
    _say("dual packed", rows, cols)
    rng = np.random.default_rng(rows * 7 + cols)
    x = _specials(wl.normal_bf16(rng, (rows, cols), outlier_frac=0.01), rng)
    xd = to_dev(x).view(torch.bfloat16)
    dev = xd.device
    pr = mx.PackedWeight(torch.full((mx.packed_bytes(1, rows, cols, 0),), 0xEE, dtype=torch.uint8, device=dev),
                         torch.full((mx.packed_bytes(1, rows, cols, 1),), 0xEE, dtype=torch.uint8, device=dev),
                         1, rows, cols)
    pc = mx.PackedWeight(torch.full((mx.packed_bytes(1, cols, rows, 0),), 0xEE, dtype=torch.uint8, device=dev),
                         torch.full((mx.packed_bytes(1, cols, rows, 1),), 0xEE, dtype=torch.uint8, device=dev),
                         1, cols, rows)
    mx.quantize_dual_packed_(xd, pr, pc)
    torch.cuda.synchronize()
    if rows * cols <= 1 << 20:
        q1, s1 = oracle_mod.quantize(x, 1)
        q0, s0 = oracle_mod.quantize(x, 0)
        qp1, sp1 = oracle_mod.pack(q1.reshape(1, rows, cols), s1.reshape(1, rows, cols // 32), 1, rows, cols)
        qp0, sp0 = oracle_mod.pack(q0.reshape(1, cols, rows), s0.reshape(1, cols, rows // 32), 1, cols, rows)
        assert np.array_equal(to_host(pr.q), qp1) and np.array_equal(to_host(pr.s), sp1)
        assert np.array_equal(to_host(pc.q), qp0) and np.array_equal(to_host(pc.s), sp0)
    else:
        qr, sr, qc, sc = mx.quantize_dual(xd)
        r1 = mx.repack(qr, sr)
        r0 = mx.repack(qc, sc)
        torch.cuda.synchronize()
        assert torch.equal(pr.q, r1.q) and torch.equal(pr.s, r1.s)
        assert torch.equal(pc.q, r0.q) and torch.equal(pc.s, r0.s)


@pytest.mark.parametrize("batch,rows,cols", [(3, 96, 160), (2, 288, 416), (128, 1536, 2048)])
def test_quantize_dual_packed_batched(mx, oracle_mod, batch, rows, cols):
    """mxfp8_quantize_dual_packed over a batch (the experts of an MoE layer):
    matrix b's packed bytes of both axes are exactly the oracle's packing of
    its own quantize (small shapes), and at the Qwen3-30B-A3B gate_up weight
    shape equal mxfp8_quantize_packed along K and mxfp8_quantize_packed_axis0."""
    import torch
    _say("dual packed batched", batch, rows, cols)
    rng = np.random.default_rng(batch * 31 + rows + cols)
    x = wl.normal_bf16(rng, (batch, rows, cols), std=0.02, outlier_frac=0.01)
    if batch * rows * cols <= 1 << 20:
        x = _specials(x.reshape(batch * rows, cols), rng).reshape(batch, rows, cols)
    xd = to_dev(x).view(torch.bfloat16)
    dev = xd.device

    def pw(n, k):
        return mx.PackedWeight(torch.full((mx.packed_bytes(batch, n, k, 0),), 0xEE, dtype=torch.uint8, device=dev),
                               torch.full((mx.packed_bytes(batch, n, k, 1),), 0xEE, dtype=torch.uint8, device=dev),
                               batch, n, k)
    pr, pc = pw(rows, cols), pw(cols, rows)
    mx.quantize_dual_packed_(xd, pr, pc)
    torch.cuda.synchronize()
    if batch * rows * cols <= 1 << 20:
        q1, s1 = oracle_mod.quantize(x.reshape(batch * rows, cols), 1)
        qp1, sp1 = oracle_mod.pack(q1.reshape(batch, rows, cols), s1.reshape(batch, rows, cols // 32),
                                   batch, rows, cols)
        qt = np.stack([oracle_mod.quantize(x[b], 0)[0] for b in range(batch)])
        st = np.stack([oracle_mod.quantize(x[b], 0)[1] for b in range(batch)])
        qp0, sp0 = oracle_mod.pack(qt, st, batch, cols, rows)
        assert np.array_equal(to_host(pr.q), qp1) and np.array_equal(to_host(pr.s), sp1)
        assert np.array_equal(to_host(pc.q), qp0) and np.array_equal(to_host(pc.s), sp0)
    else:
        r1, r0 = pw(rows, cols), pw(cols, rows)
        mx.quantize_packed_(xd, r1)
        mx.quantize_packed_axis0_(xd, r0)
        torch.cuda.synchronize()
        assert torch.equal(pr.q, r1.q) and torch.equal(pr.s, r1.s)
        assert torch.equal(pc.q, r0.q) and torch.equal(pc.s, r0.s)
