"""GPU parity of mxfp8_repack, mxfp8_gemm and mxfp8_grouped_gemm against the oracle.

Bars: repack bytes identical to the oracle's packing of the layout spec; GEMM
results bit-identical where the exact result is representable in fp32 in any
summation order (small-integer elements, narrow scales; one-hot blocks), and
|C - C_ref| <= 1e-4 * sum_k |a_k b_k| per element otherwise (bf16 outputs add
the bf16 rounding, 2^-8 |C_ref|).  Shapes span several tiles with ragged
M/N/K tails, the Qwen3-8B qkv layer at full size (sampled rows), and MoE
groups with empty and padded experts.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from conftest import sample_rows, to_dev, to_host

pytestmark = pytest.mark.gpu

E4M3_INT = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}


def _say(*a):
    print(*a, flush=True)


def _quant_pair(oracle_mod, x):
    return oracle_mod.quantize(x, 1)


def _int_operand(rng, rows, K, lo=125, hi=130):
    ints = rng.integers(-4, 5, size=(rows, K))
    mag = np.vectorize(lambda v: E4M3_INT[abs(int(v))])(ints).astype(np.uint8)
    codes = (mag | np.where(ints < 0, 0x80, 0)).astype(np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


def _hw_term(oracle_mod, aq, as_, bq, bs):
    """Per element, sum over the 128-K steps of max_k |a_k b_k| within the step
    (dequantized operands).  The MI355X FP8 matrix datapath sums each
    instruction's products with about 12 bits relative to the largest product
    (measured: at most 2^-10.8 of it per instruction), so on small-K,
    outlier-dominated data the error can exceed 1e-4 * sum|ab|; adversarial
    cases are checked against 1e-4 * sum|ab| + 2^-10 * this term."""
    M, K = aq.shape
    N = bq.shape[0]
    A = np.abs(oracle_mod.dequantize(aq, as_, M, K, 1))
    B = np.abs(oracle_mod.dequantize(bq, bs, N, K, 1))
    H = np.zeros((M, N))
    for k0 in range(0, K, 128):
        step = np.zeros((M, N))
        for k in range(k0, min(K, k0 + 128)):
            np.maximum(step, np.outer(A[:, k], B[:, k]), out=step)
        H += step
    return H


# Cap on the ratio of |C - C_ref| to the pure allowance 1e-4 * sum|ab| (+ bf16
# rounding) for the scaled-MFMA path on the adversarial inputs below.  Measured
# on MI355X: 1.013 on the 1000 x 96 x 160 fp32 case (1% x20 outliers, 5
# k-steps), 0.32-0.94 on the other ragged cases, 0.09-0.11 on the learner
# orientations; every configured workload stays below 1.
PURE_RATIO_MAX = 1.25


def _bound_with_hw(c, ref, sabs, H, out):
    err = np.abs(np.asarray(c, np.float64) - ref)
    allow = 1e-4 * sabs + 2.0 ** -10 * H
    if out == "bf16":
        allow = allow + 2.0 ** -8 * np.abs(ref)
    return bool(np.all(err <= allow)), float(np.max(err / np.maximum(allow, 1e-300)))


def _gemm_dev(mx, aq, as_, bq, bs, packed, out_dtype, accurate=False):
    a_q, a_s = to_dev(aq), to_dev(as_)
    if packed:
        w = mx.repack(to_dev(bq), to_dev(bs))
        c = mx.gemm(a_q, a_s, w, out_dtype, accurate=accurate)
    else:
        c = mx.gemm(a_q, a_s, (to_dev(bq), to_dev(bs)), out_dtype, accurate=accurate)
    torch.cuda.synchronize()
    return to_host(c.float()) if out_dtype == torch.bfloat16 else to_host(c)


@pytest.mark.parametrize("batch,N,K", [(1, 256, 128), (1, 300, 320), (3, 17, 96), (2, 512, 768),
                                       (2, 300, 384), (5, 1000, 1056), (1, 6144, 4096)])
def test_repack_matches_oracle(mx, oracle_mod, batch, N, K):
    _say("repack", batch, N, K)
    rng = np.random.default_rng(batch * N + K)
    q = rng.integers(0, 256, (batch, N, K)).astype(np.uint8)
    s = rng.integers(0, 256, (batch, N, K // 32)).astype(np.uint8)
    qp_ref, sp_ref = oracle_mod.pack(q, s, batch, N, K)
    w = mx.repack(to_dev(q), to_dev(s))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(w.q), qp_ref)
    assert np.array_equal(to_host(w.s), sp_ref)
    q2, s2 = oracle_mod.unpack(to_host(w.q), to_host(w.s), batch, N, K)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("M,N,K", [(64, 48, 512), (300, 272, 4096)])
def test_gemm_one_hot_blocks_exact(mx, oracle_mod, packed, M, N, K):
    """Only block b* of each row is non-zero: C = 32 * 2^(sa + sb - 254) exactly.
    Different b* per row / column pins the lane -> (row, K block, scale byte)
    mapping of the scaled MFMA; K = 4096 spans four 8-step scale chunks and
    two row tiles of A and of B."""
    nb = K // 32
    rng = np.random.default_rng(30)
    aq = np.zeros((M, K), np.uint8)
    bq = np.zeros((N, K), np.uint8)
    as_ = rng.integers(100, 150, (M, nb)).astype(np.uint8)
    bs = rng.integers(100, 150, (N, nb)).astype(np.uint8)
    ab = np.arange(M) % nb
    bb = (np.arange(N) * 5) % nb
    for m in range(M):
        aq[m, ab[m] * 32:(ab[m] + 1) * 32] = 0x38
    for n in range(N):
        bq[n, bb[n] * 32:(bb[n] + 1) * 32] = 0x38
    # make rows and columns that share a block meet: duplicate a few b*
    bb[:M % N] = ab[:M % N]
    bq[:] = 0
    for n in range(N):
        bq[n, bb[n] * 32:(bb[n] + 1) * 32] = 0x38
    _say("gemm one-hot", M, N, K, packed)
    c = _gemm_dev(mx, aq, as_, bq, bs, packed, torch.float32)
    ref, _ = oracle_mod.gemm(aq, as_, bq, bs)
    expect = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            if ab[m] == bb[n]:
                expect[m, n] = 32.0 * 2.0 ** (int(as_[m, ab[m]]) + int(bs[n, bb[n]]) - 254)
    assert np.array_equal(ref, expect)
    assert np.array_equal(c.astype(np.float64), expect)


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (200, 300, 416), (256, 512, 1024),
                                   (33, 17, 32), (513, 264, 4096)])
@pytest.mark.parametrize("packed", [False, True])
def test_gemm_exact_integer_cases(mx, oracle_mod, M, N, K, packed):
    rng = np.random.default_rng(M + N + K)
    aq, as_ = _int_operand(rng, M, K)
    bq, bs = _int_operand(rng, N, K)
    _say("gemm exact", M, N, K, packed)
    c = _gemm_dev(mx, aq, as_, bq, bs, packed, torch.float32)
    ref, _ = oracle_mod.gemm(aq, as_, bq, bs)
    bad = np.argwhere(c.astype(np.float64) != ref)
    assert bad.size == 0, (bad[:5], c[tuple(bad[0])], ref[tuple(bad[0])])


def test_gemm_tiny_config(mx, oracle_mod):
    d = wl.tiny(0)
    xq, xs = _quant_pair(oracle_mod, d["X"])
    wq, ws = _quant_pair(oracle_mod, d["W"])
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
    for packed in (False, True):
        _say("gemm tiny", packed)
        c = _gemm_dev(mx, xq, xs, wq, ws, packed, torch.float32)
        ok, worst = oracle_mod.gemm_bound_ok(c, ref, sabs, "f32")
        assert ok, worst


@pytest.mark.parametrize("M,N,K", [(200, 300, 416), (64, 1000, 2080), (1000, 96, 160)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_random_ragged(mx, oracle_mod, M, N, K, out):
    rng = np.random.default_rng(M * N + K)
    X = wl.normal_bf16(rng, (M, K), outlier_frac=0.01)
    W = wl.normal_bf16(rng, (N, K), std=0.02)
    xq, xs = _quant_pair(oracle_mod, X)
    wq, ws = _quant_pair(oracle_mod, W)
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
    H = _hw_term(oracle_mod, xq, xs, wq, ws)
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    cs = []
    for packed in (False, True):
        _say("gemm random", M, N, K, out, packed)
        c = _gemm_dev(mx, xq, xs, wq, ws, packed, tdt)
        ok, worst = _bound_with_hw(c, ref, sabs, H, out)
        _, pure = oracle_mod.gemm_bound_ok(c, ref, sabs, out)
        _say("  worst error / (pure bound + hardware term) %.3f, error / pure bound %.3f" % (worst, pure))
        assert ok, (packed, worst)
        assert pure <= PURE_RATIO_MAX, (packed, pure)
        cs.append(c)
    # packed and canonical B run the same arithmetic in the same order
    assert np.array_equal(cs[0], cs[1])


@pytest.mark.parametrize("M,N,K", [(200, 300, 416), (64, 1000, 2080), (1000, 96, 160), (513, 264, 4096)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_accurate_pure_bound(mx, oracle_mod, M, N, K, out):
    """mxfp8_gemm_accurate on the adversarial ragged inputs (1% x20 outliers,
    small K): every element within the pure bound 1e-4 * sum|ab| (+ bf16
    rounding), no hardware term; packed and canonical B give the same bits."""
    rng = np.random.default_rng(M * N + K)
    X = wl.normal_bf16(rng, (M, K), outlier_frac=0.01)
    W = wl.normal_bf16(rng, (N, K), std=0.02)
    xq, xs = _quant_pair(oracle_mod, X)
    wq, ws = _quant_pair(oracle_mod, W)
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    cs = []
    for packed in (False, True):
        _say("gemm accurate", M, N, K, out, packed)
        c = _gemm_dev(mx, xq, xs, wq, ws, packed, tdt, accurate=True)
        ok, worst = oracle_mod.gemm_bound_ok(c, ref, sabs, out)
        _say("  error / pure bound %.4f" % worst)
        assert ok, (packed, worst)
        cs.append(c)
    assert np.array_equal(cs[0], cs[1])


def test_gemm_accurate_outlier_products(mx, oracle_mod):
    """Single-step products dominated by outliers on both operands (2% x20
    each): the scaled-MFMA path errs by up to 2^-10 max|ab| there; the
    accurate path stays within the pure bound on every element, and its
    error is far below 2^-16 max|ab|."""
    rng = np.random.default_rng(36)
    M, N, K = 512, 256, 128
    X = wl.normal_bf16(rng, (M, K), outlier_frac=0.02)
    W = wl.normal_bf16(rng, (N, K), std=0.02, outlier_frac=0.02)
    xq, xs = _quant_pair(oracle_mod, X)
    wq, ws = _quant_pair(oracle_mod, W)
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
    H = _hw_term(oracle_mod, xq, xs, wq, ws)
    c = _gemm_dev(mx, xq, xs, wq, ws, True, torch.float32, accurate=True).astype(np.float64)
    ok, worst = oracle_mod.gemm_bound_ok(c, ref, sabs, "f32")
    _say("accurate: error / pure bound %.4f, log2 max error / max|ab| %.2f"
         % (worst, float(np.log2(np.max(np.abs(c - ref) / np.maximum(H, 1e-300)) + 1e-300))))
    assert ok, worst
    assert np.all(np.abs(c - ref) <= 2.0 ** -16 * H)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (200, 300, 416), (513, 264, 4096)])
def test_gemm_accurate_exact_cases(mx, oracle_mod, M, N, K, packed):
    """Exact results compare bit for bit on both paths: small-integer elements
    with narrow scales (the folded conversion), and with scale codes at the
    ends of the E8M0 range (A in {0, 1, 2, 250, 251, 252}, B chosen so that
    every block's combined exponent stays within [-8, 8]: the accurate path's
    per-block fallback for codes outside [3, 246]; the result is exact in
    fp32 either way)."""
    rng = np.random.default_rng(M + N + K + 7)
    aq, as_ = _int_operand(rng, M, K)
    bq, bs = _int_operand(rng, N, K)
    _say("gemm accurate exact", M, N, K, packed)
    ref, _ = oracle_mod.gemm(aq, as_, bq, bs)
    c = _gemm_dev(mx, aq, as_, bq, bs, packed, torch.float32, accurate=True)
    assert np.array_equal(c.astype(np.float64), ref)
    # end-of-range scale codes: per block, A low and B high, or A high and B low
    nb = K // 32
    lowhi = rng.integers(0, 2, size=nb).astype(bool)
    as2 = np.where(lowhi[None, :], rng.integers(0, 3, size=(M, nb)), rng.integers(250, 253, size=(M, nb)))
    bs2 = np.where(lowhi[None, :], rng.integers(250, 253, size=(N, nb)), rng.integers(3, 6, size=(N, nb)))
    as2, bs2 = as2.astype(np.uint8), bs2.astype(np.uint8)
    ref2, _ = oracle_mod.gemm(aq, as2, bq, bs2)
    c2 = _gemm_dev(mx, aq, as2, bq, bs2, packed, torch.float32, accurate=True)
    assert np.array_equal(c2.astype(np.float64), ref2)
    c3 = _gemm_dev(mx, aq, as2, bq, bs2, packed, torch.float32)
    assert np.array_equal(c3.astype(np.float64), ref2)


@pytest.mark.parametrize("M,N,K,out", [(500, 32968, 160, "f32"), (512, 32768, 256, "bf16"),
                                       (4000, 6100, 512, "bf16"), (4096, 6144, 1024, "f32")])
def test_gemm_mixed_tiles_full_output(mx, oracle_mod, M, N, K, out):
    """Shapes whose tile count leaves a partial round of 256x256 tiles launch
    256x256 tiles over the leading columns and 256x128 tiles over the rest in
    one grid (the qkv layer's launch form).  Every element is checked, with
    ragged M and N tails and K either a multiple of 128 or not.  With as many
    small tiles as large ones, packed B and K % 512 == 0 (the last two
    shapes) a workgroup computes one tile of each kind; its output must equal
    the one-tile-per-workgroup launch of canonical B bit for bit."""
    rng = np.random.default_rng(M + N + K)
    X = wl.normal_bf16(rng, (M, K))
    W = wl.normal_bf16(rng, (N, K), std=0.02)
    xq, xs = _quant_pair(oracle_mod, X)
    wq, ws = _quant_pair(oracle_mod, W)
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    cs = []
    for packed in (False, True):
        _say("gemm mixed tiles", M, N, K, out, packed)
        c = _gemm_dev(mx, xq, xs, wq, ws, packed, tdt)
        ok, worst = oracle_mod.gemm_bound_ok(c, ref, sabs, out)
        assert ok, (packed, worst)
        cs.append(c)
    assert np.array_equal(cs[0], cs[1])


def test_gemm_dgrad_wgrad_orientations(mx, oracle_mod):
    """The learner's three GEMMs through one A*B^T: fprop (X, W along K),
    dgrad (dY along N, W quantized with axis 0), wgrad (dY, X along tokens)."""
    rng = np.random.default_rng(31)
    T, H, O = 256, 192, 320
    X = wl.normal_bf16(rng, (T, H))
    W = wl.normal_bf16(rng, (O, H), std=0.02)
    dY = wl.normal_bf16(rng, (T, O), std=2.0 ** -10)
    cases = {
        "fprop": (oracle_mod.quantize(X, 1), oracle_mod.quantize(W, 1)),     # [T,H] x [O,H]^T
        "dgrad": (oracle_mod.quantize(dY, 1), oracle_mod.quantize(W, 0)),    # [T,O] x [H,O]^T
        "wgrad": (oracle_mod.quantize(dY, 0), oracle_mod.quantize(X, 0)),    # [O,T] x [H,T]^T
    }
    for name, ((aq, as_), (bq, bs)) in cases.items():
        _say("gemm", name)
        ref, sabs = oracle_mod.gemm(aq, as_, bq, bs)
        c = _gemm_dev(mx, aq, as_, bq, bs, False, torch.float32)
        ok, worst = _bound_with_hw(c, ref, sabs, _hw_term(oracle_mod, aq, as_, bq, bs), "f32")
        _, pure = oracle_mod.gemm_bound_ok(c, ref, sabs, "f32")
        _say("  worst error / (pure bound + hardware term) %.3f, error / pure bound %.3f" % (worst, pure))
        assert ok, (name, worst)
        assert pure <= PURE_RATIO_MAX, (name, pure)


def test_gemm_qkv_full_output(mx, oracle_mod):
    """The Qwen3-8B qkv layer (4096 x 6144 x 4096, bf16 out) in the launch the
    bench times: every one of the 25.2M outputs against the oracle."""
    d = wl.qkv(0)
    xq, xs = _quant_pair(oracle_mod, d["X"])
    wq, ws = _quant_pair(oracle_mod, d["W"])
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
    _say("gemm qkv full output")
    c = _gemm_dev(mx, xq, xs, wq, ws, True, torch.bfloat16)
    ok, worst = oracle_mod.gemm_bound_ok(c, ref, sabs, "bf16")
    _say("qkv worst error / allowance", worst)
    assert ok, worst
    _say("gemm qkv full output, accurate path")
    ca = _gemm_dev(mx, xq, xs, wq, ws, True, torch.bfloat16, accurate=True)
    ok, worst_a = oracle_mod.gemm_bound_ok(ca, ref, sabs, "bf16")
    _say("qkv accurate worst error / allowance", worst_a)
    assert ok, worst_a
    del ca
    # both operands packed, A quantized straight from the BF16 activations:
    # the same bits as the canonical-A launch above
    _say("gemm qkv full output, packed A")
    Aq, _, _ = mx.quantize_packed(to_dev(d["X"]).view(torch.bfloat16), canonical=False)
    P = mx.repack(to_dev(wq), to_dev(ws))
    cp = to_host(mx.gemm_packed(Aq, P, torch.bfloat16).float())
    assert np.array_equal(cp, c)
    del cp
    # the page's healthy-kernel error band for a dense layer: relative error
    # of the MXFP8 layer against the high-precision GEMM on the BF16 inputs
    rows = sample_rows(xq.shape[0], 256, 256, 32)
    from workloads import bf16_bits_to_f32
    xf = bf16_bits_to_f32(d["X"][rows]).astype(np.float64)
    wf = bf16_bits_to_f32(d["W"]).astype(np.float64)
    y = xf @ wf.T
    rel = np.linalg.norm(c[rows] - y) / np.linalg.norm(y)
    assert 0.005 < rel < 0.25, rel


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (200, 300, 512), (1000, 96, 1024), (513, 264, 4096),
                                   (2048, 9216, 512), (512, 32768, 256), (4096, 9216, 512), (3072, 9216, 512),
                                   (4096, 6140, 512), (300, 4100, 384), (1, 8, 128), (33, 4, 128),
                                   (512, 6144, 4096), (100, 264, 512), (640, 1024, 1024), (129, 8, 128)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_packed_a_matches_canonical(mx, oracle_mod, M, N, K, out):
    """mxfp8_gemm_packed: A quantized straight into the packed layout
    (mxfp8_quantize_packed) gives the same bytes as repacking the canonical
    grid, and the GEMM over it is bit-identical to mxfp8_gemm with canonical
    A, over every kernel the launcher picks: the copying/computing-wave
    kernel with 128-row tiles (the few-tile shapes: 512x6144, 100x264,
    640x1024, 129x8, 1000x96, 513x264, 64x256, 1x8, 33x4, and 200x300 and
    300x4100 with fp32 output) or 256x128 tiles (2048x9216), and otherwise
    the 256x256 tiles (3072x9216, and 512x32768 where 256x128 tiles would
    take two rounds), the mixed launch (4096x9216: 32 large + 8 small tile
    columns), the paired launch (4096x6140 bf16: N % 8 != 0) and 256x128
    tiles (300x4100 bf16); the smaller cases also against the oracle."""
    rng = np.random.default_rng(M * 7 + N + K)
    x = wl.normal_bf16(rng, (M, K))
    w = wl.normal_bf16(rng, (N, K), std=0.02)
    xq, xs = _quant_pair(oracle_mod, x)
    wq, ws = _quant_pair(oracle_mod, w)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    _say("gemm packed A", M, N, K, out)
    P = mx.repack(to_dev(wq), to_dev(ws))
    c0 = mx.gemm(to_dev(xq), to_dev(xs), P, dt)
    Ar = mx.repack(to_dev(xq), to_dev(xs))
    Aq, _, _ = mx.quantize_packed(to_dev(x).view(torch.bfloat16), canonical=False)
    assert torch.equal(Ar.q, Aq.q) and torch.equal(Ar.s, Aq.s)
    c1 = mx.gemm_packed(Aq, P, dt)
    torch.cuda.synchronize()
    iv = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(c0.view(iv), c1.view(iv))
    if M * N * K <= 2 ** 28:
        ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
        ok, worst = oracle_mod.gemm_bound_ok(to_host(c1.float()) if out == "bf16" else to_host(c1), ref, sabs, out)
        assert ok, worst


def test_gemm_deterministic(mx, oracle_mod):
    rng = np.random.default_rng(33)
    xq, xs = _quant_pair(oracle_mod, wl.normal_bf16(rng, (512, 1024)))
    wq, ws = _quant_pair(oracle_mod, wl.normal_bf16(rng, (768, 1024), std=0.02))
    a_q, a_s = to_dev(xq), to_dev(xs)
    w = mx.repack(to_dev(wq), to_dev(ws))
    c0 = mx.gemm(a_q, a_s, w, torch.float32)
    for _ in range(10):
        assert torch.equal(mx.gemm(a_q, a_s, w, torch.float32), c0)


def _moe_case(oracle_mod, G, N, K, tokens, topk, seed, empty=()):
    rng = np.random.default_rng(seed)
    route = wl.zipf_topk_routing(rng, tokens, G, topk)
    for e in empty:
        route[route == e] = (e + 1) % G
    off, row_token, counts = wl.group_layout(route, G)
    X = wl.normal_bf16(rng, (tokens, K))
    A = np.zeros((row_token.size, K), np.uint16)
    A[row_token >= 0] = X[row_token[row_token >= 0]]
    aq, as_ = oracle_mod.quantize(A, 1)
    W = wl.normal_bf16(rng, (G, N, K), std=0.02)
    bq = np.empty((G, N, K), np.uint8)
    bs = np.empty((G, N, K // 32), np.uint8)
    for g in range(G):
        bq[g], bs[g] = oracle_mod.quantize(W[g], 1)
    return aq, as_, bq, bs, off, row_token


@pytest.mark.parametrize("G,N,K,tokens,topk", [(8, 256, 256, 300, 2), (5, 200, 160, 97, 3),
                                               (16, 512, 768, 1024, 4),
                                               # groups of 256+ rows: the persistent launch, more
                                               # tiles than CUs (K % 512 != 0 and == 0)
                                               (8, 1024, 768, 8192, 2), (8, 1024, 1024, 8192, 2),
                                               (4, 200, 512, 2048, 2)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_grouped_gemm_small(mx, oracle_mod, G, N, K, tokens, topk, out):
    aq, as_, bq, bs, off, row_token = _moe_case(oracle_mod, G, N, K, tokens, topk, G + N,
                                                empty=(1,))
    ref, sabs, grp = oracle_mod.grouped_gemm(aq, as_, bq, bs, off)
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    w = mx.repack(to_dev(bq), to_dev(bs))
    M = aq.shape[0]
    sentinel = torch.full((M + 64, N), 7.0, dtype=tdt, device="cuda")
    _say("grouped", G, N, K, tokens, out)
    c = mx.grouped_gemm(to_dev(aq), to_dev(as_), w, to_dev(off), tdt, out=sentinel[:M])
    torch.cuda.synchronize()
    ch = to_host(sentinel.float())
    ok, worst = oracle_mod.gemm_bound_ok(ch[:M], ref, sabs, out)
    assert ok, worst
    assert np.all(ch[M:] == 7.0)                 # nothing written past M_total
    assert np.all(ch[:M][row_token < 0] == 0.0)  # zero padding rows give zero rows
    assert c.data_ptr() == sentinel.data_ptr()


def test_grouped_gemm_untouched_rows_outside_groups(mx, oracle_mod):
    G, N, K = 4, 128, 128
    rng = np.random.default_rng(34)
    M = 256
    aq, as_ = oracle_mod.quantize(wl.normal_bf16(rng, (M, K)), 1)
    W = wl.normal_bf16(rng, (G, N, K), std=0.02)
    bq = np.stack([oracle_mod.quantize(W[g], 1)[0] for g in range(G)])
    bs = np.stack([oracle_mod.quantize(W[g], 1)[1] for g in range(G)])
    off = np.array([32, 64, 64, 160, 192], np.int32)      # rows [0,32) and [192,256) in no group
    ref, sabs, grp = oracle_mod.grouped_gemm(aq, as_, bq, bs, off)
    w = mx.repack(to_dev(bq), to_dev(bs))
    out = torch.full((M, N), -3.0, dtype=torch.float32, device="cuda")
    _say("grouped untouched rows")
    mx.grouped_gemm(to_dev(aq), to_dev(as_), w, to_dev(off), torch.float32, out=out)
    ch = to_host(out)
    inside = grp >= 0
    ok, worst = oracle_mod.gemm_bound_ok(ch[inside], ref[inside], sabs[inside], "f32")
    assert ok, worst
    assert np.all(ch[~inside] == -3.0)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_grouped_gemm_persistent_rows_outside_groups(mx, oracle_mod, out):
    """The 256-row persistent grouped launch (M_total >= 256 G) with rows in
    no group ([0, 64) and [960, 1024)) and an empty group: those rows
    untouched, every group row within the bound."""
    G, N, K = 3, 264, 384
    rng = np.random.default_rng(35)
    M = 1024
    aq, as_ = oracle_mod.quantize(wl.normal_bf16(rng, (M, K)), 1)
    W = wl.normal_bf16(rng, (G, N, K), std=0.02)
    bq = np.stack([oracle_mod.quantize(W[g], 1)[0] for g in range(G)])
    bs = np.stack([oracle_mod.quantize(W[g], 1)[1] for g in range(G)])
    off = np.array([64, 320, 320, 960], np.int32)
    ref, sabs, grp = oracle_mod.grouped_gemm(aq, as_, bq, bs, off)
    w = mx.repack(to_dev(bq), to_dev(bs))
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    res = torch.full((M, N), -3.0, dtype=tdt, device="cuda")
    _say("grouped persistent untouched rows", out)
    mx.grouped_gemm(to_dev(aq), to_dev(as_), w, to_dev(off), tdt, out=res)
    ch = to_host(res.float())
    inside = grp >= 0
    ok, worst = oracle_mod.gemm_bound_ok(ch[inside], ref[inside], sabs[inside], out)
    assert ok, worst
    assert np.all(ch[~inside] == -3.0)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_gemm_moe_full_size_sampled(mx, oracle_mod, proj):
    """The Qwen3-30B-A3B expert GEMMs at full size (8192 tokens, top-8
    Zipf(1.1) routing, 128 experts, groups padded to 32): gate_up
    [67616 x 1536 x 2048] and down [67616 x 2048 x 768] in the launch the
    bench times, checked on 512 rows that include one row of every
    non-empty expert."""
    d = wl.moe(0)
    A = d["A_gu"] if proj == "gate_up" else d["A_d"]
    Wt = d["W_gu"] if proj == "gate_up" else d["W_d"]
    aq, as_ = oracle_mod.quantize(A, 1)
    G, N, K = Wt.shape
    bq = np.empty((G, N, K), np.uint8)
    bs = np.empty((G, N, K // 32), np.uint8)
    for g in range(G):
        bq[g], bs[g] = oracle_mod.quantize(Wt[g], 1)
    rows = sample_rows(aq.shape[0], 256, 512, 35, groups=d["offsets"])
    ref, sabs, grp = oracle_mod.grouped_gemm(aq, as_, bq, bs, d["offsets"], rows=rows)
    assert np.all(grp >= 0)
    assert np.unique(grp).size == int(np.count_nonzero(np.diff(d["offsets"])))
    w = mx.repack(to_dev(bq), to_dev(bs))
    _say("grouped MoE full size", proj, aq.shape, N)
    c = mx.grouped_gemm(to_dev(aq), to_dev(as_), w, to_dev(d["offsets"]), torch.bfloat16)
    ch = to_host(c.float())
    ok, worst = oracle_mod.gemm_bound_ok(ch[rows], ref, sabs, "bf16")
    _say("moe", proj, "worst error / allowance", worst)
    assert ok, worst


def test_mfma_accumulation_error_model(mx, oracle_mod):
    """The hardware term used above, pinned on its own: over many random
    128-K single-step products with outliers, |C - C_ref| stays within
    2^-10 * max_k |a_k b_k| (and the pure spec bound holds whenever the
    products are not dominated by a few terms)."""
    rng = np.random.default_rng(36)
    M, N, K = 512, 256, 128
    X = wl.normal_bf16(rng, (M, K), outlier_frac=0.02)
    W = wl.normal_bf16(rng, (N, K), std=0.02, outlier_frac=0.02)
    xq, xs = _quant_pair(oracle_mod, X)
    wq, ws = _quant_pair(oracle_mod, W)
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
    H = _hw_term(oracle_mod, xq, xs, wq, ws)
    c = _gemm_dev(mx, xq, xs, wq, ws, True, torch.float32).astype(np.float64)
    err = np.abs(c - ref)
    ratio = err / np.maximum(H, 1e-300)
    _say("mfma error / max|ab| (log2):", float(np.log2(ratio.max() + 1e-300)))
    assert np.all(err <= 2.0 ** -10 * H)
    spread = sabs >= 8 * H          # sums not dominated by a few products
    assert np.all(err[spread] <= 1e-4 * sabs[spread])


def test_gemm_mlp_step_full_size_sampled(mx, oracle_mod):
    """Qwen3-8B MLP micro-batch of 8192 tokens: the six GEMMs of forward, data
    gradient and weight gradient at full size, in the launch configuration the
    library picks for them, each checked on 256 sampled output rows (one in
    every 256-row tile) against the oracle (operands quantized by the oracle)
    with the 1e-4 * sum|ab| bound."""
    d = wl.mlp(0)
    q = {}
    for name, axis in (("X", 1), ("h", 1), ("W_gu", 1), ("W_d", 1), ("dY_gu", 1), ("dY_d", 1),
                       ("W_gu", 0), ("W_d", 0), ("X", 0), ("h", 0), ("dY_gu", 0), ("dY_d", 0)):
        q[(name, axis)] = oracle_mod.quantize(d[name], axis)
    gemms = [
        ("fprop gate_up", ("X", 1), ("W_gu", 1), True, "bf16"),
        ("fprop down", ("h", 1), ("W_d", 1), True, "bf16"),
        ("dgrad gate_up", ("dY_gu", 1), ("W_gu", 0), False, "bf16"),
        ("dgrad down", ("dY_d", 1), ("W_d", 0), False, "bf16"),
        ("wgrad gate_up", ("dY_gu", 0), ("X", 0), False, "f32"),
        ("wgrad down", ("dY_d", 0), ("h", 0), False, "f32"),
    ]
    for i, (name, ka, kb, packed, out) in enumerate(gemms):
        aq, as_ = q[ka]
        bq, bs = q[kb]
        rows = sample_rows(aq.shape[0], 256, 256, 37 + i)
        _say("mlp", name, aq.shape, bq.shape)
        ref, sabs = oracle_mod.gemm(aq, as_, bq, bs, rows=rows)
        tdt = torch.float32 if out == "f32" else torch.bfloat16
        c = _gemm_dev(mx, aq, as_, bq, bs, packed, tdt)
        ok, worst = oracle_mod.gemm_bound_ok(c[rows], ref, sabs, out)
        _say("mlp", name, "rows", rows.size, "worst error / allowance", worst)
        assert ok, (name, worst)
        del c


@pytest.mark.parametrize("M,N,K,out", [(64, 256, 1024, "bf16"), (200, 300, 2080, "f32"), (1000, 96, 4128, "bf16"),
                                       (32, 4096, 12288, "f32"), (512, 6144, 4096, "bf16")])
def test_gemm_splitk_matches_oracle(mx, oracle_mod, M, N, K, out):
    """mxfp8_gemm_splitk: K split over workgroups for shapes with few tiles,
    partials summed in slice order.  Every element within the GEMM bound, for
    packed and canonical B (identical bits: same arithmetic), the last slice
    unaligned when K % 128 != 0; two calls give the same bits; a workspace too
    small for the full split still gives a correct result, and no workspace
    gives exactly mxfp8_gemm's result."""
    import torch
    _say("gemm splitk", M, N, K, out, mx.gemm_splitk_workspace_bytes(M, N, K))
    assert mx.gemm_splitk_workspace_bytes(M, N, K) > 0
    rng = np.random.default_rng(M + N + K)
    X = wl.normal_bf16(rng, (M, K))
    W = wl.normal_bf16(rng, (N, K), std=0.02)
    xq, xs = _quant_pair(oracle_mod, X)
    wq, ws = _quant_pair(oracle_mod, W)
    rows = None if M * N <= 1 << 20 else np.sort(rng.choice(M, 48, replace=False))
    ref, sabs = oracle_mod.gemm(xq, xs, wq, ws, rows=rows)
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    a_q, a_s = to_dev(xq), to_dev(xs)
    packed = mx.repack(to_dev(wq), to_dev(ws))
    canon = (to_dev(wq), to_dev(ws))

    def host(c):
        torch.cuda.synchronize()
        return to_host(c.float()) if out == "bf16" else to_host(c)

    c1 = host(mx.gemm(a_q, a_s, packed, tdt, split_k=True))
    sel = c1 if rows is None else c1[rows]
    ok, worst = oracle_mod.gemm_bound_ok(sel, ref, sabs, out)
    assert ok, worst
    assert np.array_equal(c1, host(mx.gemm(a_q, a_s, canon, tdt, split_k=True)))
    assert np.array_equal(c1, host(mx.gemm(a_q, a_s, packed, tdt, split_k=True)))
    half = torch.empty(mx.gemm_splitk_workspace_bytes(M, N, K) // 2 + 16, dtype=torch.uint8, device=a_q.device)
    c2 = host(mx.gemm(a_q, a_s, packed, tdt, workspace=half))
    ok, worst = oracle_mod.gemm_bound_ok(c2 if rows is None else c2[rows], ref, sabs, out)
    assert ok, worst
    none = torch.empty(0, dtype=torch.uint8, device=a_q.device)
    assert np.array_equal(host(mx.gemm(a_q, a_s, packed, tdt, workspace=none)), host(mx.gemm(a_q, a_s, packed, tdt)))


def _packed_split_declined(M, N, K, out):
    """Where mxfp8_gemm_packed_splitk keeps the unsplit launch although the
    split plan has slices: the launcher's 128-row tiles (they take fewer
    rounds, weighted by a k-step's copy time, than 256x128 or 256x256 tiles)
    filling at least half the CUs over at most 64 k-steps."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    es = 4 if out == "f32" else 2
    cd = lambda a, b: -(-a // b)
    full = cd(M, 256) * cd(N, 128)
    if N % (8 if es == 2 else 4) or 128 * N * es >= 2 ** 31 or full > 3 * cus:
        return False
    t_full = cd(full, cus)
    t_half = 0.67 * cd(cd(M, 128) * cd(N, 128), cus)
    t_big = 1.5 * cd(cd(M, 256) * cd(N, 256), cus)
    if (t_big < t_full - 1e-9 and t_big < t_half - 1e-9) or not t_half < t_full - 1e-9:
        return False
    return 2 * cd(M, 128) * cd(N, 128) >= cus and cd(K, 128) <= 64


@pytest.mark.parametrize("M,N,K,out", [(64, 256, 1024, "bf16"), (300, 4096, 4096, "f32"), (512, 6144, 4096, "bf16"),
                                       (512, 4096, 12288, "bf16"), (32, 1000, 2048, "f32"), (512, 1002, 1024, "bf16"),
                                       (512, 4096, 4096, "f32"), (384, 4096, 8192, "bf16")])
def test_gemm_packed_splitk_matches_canonical_split(mx, oracle_mod, M, N, K, out):
    """mxfp8_gemm_packed_splitk: the copying/computing-wave launch over
    (tile, K slice) units, fp32 partials summed in slice order.  Bit-identical
    to mxfp8_gemm_splitk over the canonical grids (the same slices and
    per-slice products), with the full workspace and with one too small for
    the full split (fewer slices, the same fitted plan on both sides); N % 4
    != 0 (512x1002) and no workspace fall back to mxfp8_gemm_packed exactly;
    the smaller shapes also against the oracle."""
    import torch
    _say("gemm packed splitk", M, N, K, out, mx.gemm_splitk_workspace_bytes(M, N, K))
    rng = np.random.default_rng(M * 3 + N + K)
    X = wl.normal_bf16(rng, (M, K))
    W = wl.normal_bf16(rng, (N, K), std=0.02)
    xq, xs = _quant_pair(oracle_mod, X)
    wq, ws = _quant_pair(oracle_mod, W)
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    a_q, a_s = to_dev(xq), to_dev(xs)
    B = mx.repack(to_dev(wq), to_dev(ws))
    A = mx.repack(a_q, a_s)

    def host(c):
        torch.cuda.synchronize()
        return to_host(c.float()) if out == "bf16" else to_host(c)

    need = mx.gemm_splitk_workspace_bytes(M, N, K)
    assert need > 0
    full = torch.empty(need, dtype=torch.uint8, device=a_q.device)
    c1 = host(mx.gemm_packed(A, B, tdt, workspace=full))
    if _packed_split_declined(M, N, K, out):
        # 128-row tiles filling half the CUs over <= 64 k-steps run unsplit:
        # bit-identical to the unsplit canonical-A GEMM
        assert np.array_equal(c1, host(mx.gemm(a_q, a_s, B, tdt)))
    elif N % 4 == 0:
        assert np.array_equal(c1, host(mx.gemm(a_q, a_s, B, tdt, workspace=full)))
        half = torch.empty(need // 2 + 16, dtype=torch.uint8, device=a_q.device)
        assert np.array_equal(host(mx.gemm_packed(A, B, tdt, workspace=half)),
                              host(mx.gemm(a_q, a_s, B, tdt, workspace=half)))
    else:
        assert np.array_equal(c1, host(mx.gemm_packed(A, B, tdt)))
    none = torch.empty(0, dtype=torch.uint8, device=a_q.device)
    assert np.array_equal(host(mx.gemm_packed(A, B, tdt, workspace=none)), host(mx.gemm_packed(A, B, tdt)))
    assert np.array_equal(host(mx.gemm_packed(A, B, tdt, workspace=full)), c1)       # deterministic
    if M * N * K <= 2 ** 31:
        ref, sabs = oracle_mod.gemm(xq, xs, wq, ws)
        ok, worst = oracle_mod.gemm_bound_ok(c1, ref, sabs, out)
        assert ok, worst


@pytest.mark.parametrize("G,N,K,tokens,topk", [(8, 256, 256, 300, 2), (16, 512, 768, 1024, 4),
                                               (8, 1024, 768, 8192, 2), (4, 200, 512, 2048, 2),
                                               (4, 132, 384, 1024, 2)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_grouped_gemm_packed_a_matches_canonical(mx, oracle_mod, G, N, K, tokens, topk, out):
    """mxfp8_grouped_gemm_packed: A quantized straight into the packed layout
    (groups starting anywhere inside a panel, an empty group) gives C
    bit-identical to mxfp8_grouped_gemm over the canonical grid, and leaves
    rows past M_total untouched.  N = 132 with bf16 output takes the
    persistent 256x256 launch (the copying / computing-wave launch needs
    N % 8 == 0 for bf16), every other case the latter."""
    aq, as_, bq, bs, off, row_token = _moe_case(oracle_mod, G, N, K, tokens, topk, G + N + 1, empty=(1,))
    tdt = torch.float32 if out == "f32" else torch.bfloat16
    w = mx.repack(to_dev(bq), to_dev(bs))
    M = aq.shape[0]
    _say("grouped packed A", G, N, K, tokens, out)
    A = mx.repack(to_dev(aq), to_dev(as_))
    offs = to_dev(off)
    c0 = mx.grouped_gemm(to_dev(aq), to_dev(as_), w, offs, tdt)
    sentinel = torch.full((M + 64, N), 7.0, dtype=tdt, device="cuda")
    c1 = mx.grouped_gemm_packed(A, w, offs, tdt, out=sentinel[:M])
    torch.cuda.synchronize()
    iv = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(c0.view(iv), c1.view(iv))
    assert bool(torch.all(sentinel[M:] == 7.0))


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_gemm_packed_a_moe_full_size(mx, oracle_mod, proj):
    """The Qwen3-30B-A3B expert GEMMs at full size with packed A (the bench's
    MoE step): every output bit-identical to the canonical-A grouped GEMM."""
    d = wl.moe(0)
    A = d["A_gu"] if proj == "gate_up" else d["A_d"]
    W = d["W_gu"] if proj == "gate_up" else d["W_d"]
    G, N, K = W.shape
    _say("grouped packed A full size", proj)
    Ad = to_dev(A).view(torch.bfloat16)
    aq, as_ = mx.quantize(Ad, 1)
    Ap = mx.PackedWeight(torch.empty(mx.packed_bytes(1, A.shape[0], K, 0), dtype=torch.uint8, device="cuda"),
                         torch.empty(mx.packed_bytes(1, A.shape[0], K, 1), dtype=torch.uint8, device="cuda"),
                         1, A.shape[0], K)
    mx.quantize_many_layouts_([(Ad, Ap)])
    Wd = to_dev(W.reshape(G * N, K)).view(torch.bfloat16)
    wq, ws = mx.quantize(Wd, 1)
    w = mx.repack(wq.view(G, N, K), ws.view(G, N, K // 32))
    offs = torch.from_numpy(d["offsets"]).cuda()
    c0 = mx.grouped_gemm(aq, as_, w, offs, torch.bfloat16)
    c1 = mx.grouped_gemm_packed(Ap, w, offs, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(c0.view(torch.int16), c1.view(torch.int16))
