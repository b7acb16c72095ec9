"""Pins of the oracle's GEMM, grouped GEMM and packed layout (CPU only).

The GEMM oracle (a plain fp64 loop over dequantized operands) is checked
against exact integer arithmetic, the closed form of one-hot block products,
numpy's float64 matmul (an independent library routine), and the grouped
oracle against per-group dense products.  The packed layout is pinned by
offsets worked by hand from its written specification and by the round trip.
"""
import numpy as np
import pytest

from workloads import group_layout, normal_bf16, zipf_topk_routing

E4M3_INT = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}   # exact small integers


def _int_operand(rng, rows, K):
    ints = rng.integers(-4, 5, size=(rows, K))
    codes = np.vectorize(lambda v: E4M3_INT[abs(int(v))] | (0x80 if v < 0 else 0))(ints).astype(np.uint8)
    scales = rng.integers(125, 130, size=(rows, K // 32)).astype(np.uint8)
    return ints, codes, scales


@pytest.mark.parametrize("M,N,K", [(7, 5, 32), (33, 17, 96), (64, 48, 512)])
def test_gemm_exact_integer_case(oracle_mod, M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    ai, aq, as_ = _int_operand(rng, M, K)
    bi, bq, bs = _int_operand(rng, N, K)
    c, sabs = oracle_mod.gemm(aq, as_, bq, bs)
    # exact: sum_k a*2^(sa-127) * b*2^(sb-127), times 2^4 is an integer
    ea = np.repeat(as_.astype(np.int64) - 127, 32, axis=1)   # [-2, 2]
    eb = np.repeat(bs.astype(np.int64) - 127, 32, axis=1)
    ref16 = np.zeros((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            tot = 0
            for k in range(K):
                tot += int(ai[m, k]) * int(bi[n, k]) * (1 << (ea[m, k] + eb[n, k] + 4))
            ref16[m, n] = tot
    assert np.array_equal((c * 16).astype(np.int64), ref16.astype(np.int64))
    assert np.all(c * 16 == (c * 16).astype(np.int64))


def test_gemm_one_hot_block(oracle_mod):
    K = 256
    for bstar in (0, 3, 7):
        for sa, sb in ((127, 127), (120, 131), (200, 60)):
            aq = np.zeros((1, K), np.uint8)
            bq = np.zeros((1, K), np.uint8)
            aq[0, bstar * 32:(bstar + 1) * 32] = 0x38
            bq[0, bstar * 32:(bstar + 1) * 32] = 0x38
            as_ = np.full((1, K // 32), 127, np.uint8)
            bs = np.full((1, K // 32), 127, np.uint8)
            as_[0, bstar] = sa
            bs[0, bstar] = sb
            c, _ = oracle_mod.gemm(aq, as_, bq, bs)
            assert c[0, 0] == 32.0 * 2.0 ** (sa + sb - 254)


def test_gemm_matches_numpy_on_dequantized(oracle_mod):
    rng = np.random.default_rng(11)
    X = normal_bf16(rng, (64, 256))
    W = normal_bf16(rng, (96, 256), std=0.02)
    aq, as_ = oracle_mod.quantize(X, 1)
    bq, bs = oracle_mod.quantize(W, 1)
    A = oracle_mod.dequantize(aq, as_, 64, 256, 1)
    B = oracle_mod.dequantize(bq, bs, 96, 256, 1)
    c, sabs = oracle_mod.gemm(aq, as_, bq, bs)
    ref = A @ B.T
    assert np.all(np.abs(c - ref) <= 1e-12 * (np.abs(A) @ np.abs(B).T))
    assert np.allclose(sabs, np.abs(A) @ np.abs(B).T, rtol=1e-12, atol=0)
    rows = np.array([5, 0, 63])
    c2, s2 = oracle_mod.gemm(aq, as_, bq, bs, rows=rows)
    assert np.array_equal(c2, c[rows]) and np.array_equal(s2, sabs[rows])


def test_gemm_bound_helper_rejects_planted_error(oracle_mod):
    rng = np.random.default_rng(12)
    aq, as_ = oracle_mod.quantize(normal_bf16(rng, (32, 128)), 1)
    bq, bs = oracle_mod.quantize(normal_bf16(rng, (16, 128)), 1)
    c, sabs = oracle_mod.gemm(aq, as_, bq, bs)
    ok, _ = oracle_mod.gemm_bound_ok(c.astype(np.float32), c, sabs)
    assert ok
    bad = c.copy()
    bad[3, 4] += 2e-4 * sabs[3, 4]
    ok, worst = oracle_mod.gemm_bound_ok(bad, c, sabs)
    assert not ok and worst > 1.0


def test_grouped_gemm_equals_per_group_dense(oracle_mod):
    rng = np.random.default_rng(13)
    G, N, K, tokens = 6, 40, 96, 50
    route = zipf_topk_routing(rng, tokens, G, 2)
    off, row_token, counts = group_layout(route, G)
    X = normal_bf16(rng, (tokens, K))
    A = np.zeros((row_token.size, K), np.uint16)
    A[row_token >= 0] = X[row_token[row_token >= 0]]
    aq, as_ = oracle_mod.quantize(A, 1)
    W = normal_bf16(rng, (G, N, K), std=0.02)
    bq = np.empty((G, N, K), np.uint8)
    bs = np.empty((G, N, K // 32), np.uint8)
    for g in range(G):
        bq[g], bs[g] = oracle_mod.quantize(W[g], 1)
    c, sabs, grp = oracle_mod.grouped_gemm(aq, as_, bq, bs, off)
    assert np.all(off % 32 == 0)
    for g in range(G):
        lo, hi = off[g], off[g + 1]
        if hi == lo:
            continue
        cg, _ = oracle_mod.gemm(aq[lo:hi], as_[lo:hi], bq[g], bs[g])
        assert np.array_equal(c[lo:hi], cg)
        assert np.all(grp[lo:hi] == g)
    pad = row_token < 0
    assert np.all(c[pad] == 0.0)   # zero padding rows give exactly zero rows


def test_packed_layout_hand_offsets(oracle_mod):
    # N=300, K=320: NP = 2 panels, KS = 3 k-steps.
    N, K = 300, 320
    q = np.zeros((1, N, K), np.uint8)
    s = np.full((1, N, K // 32), 127, np.uint8)
    q[0, 17, 130] = 0xAB          # panel 0, kstep 1, row 17, chunk 0 -> slot 0^(17%8)=1
    s[0, 17, 5] = 0x42            # panel 0, kstep 1, atom 1, lane 1+16*1=17
    s[0, 299, 9] = 0x43           # panel 1, kstep 2, atom 2 (row 43), lane 11+16*1=27
    q[0, 299, 319] = 0xCD         # panel 1, row 43, kstep 2, chunk 3 -> slot 3^(43%8)=3^3=0
    qp, sp = oracle_mod.pack(q, s, 1, N, K)
    assert qp.size == 2 * 3 * 256 * 128 and sp.size == 2 * 3 * 16 * 64
    assert qp[(1 * 256 + 17) * 128 + 16 + 2] == 0xAB
    assert sp[((0 * 3 + 1) * 16 + 1) * 64 + 17] == 0x42
    assert sp[((1 * 3 + 2) * 16 + 2) * 64 + 27] == 0x43
    off = ((1 * 3 + 2) * 256 + 43) * 128 + 0 * 16 + 15
    assert qp[off] == 0xCD
    assert int((qp != 0).sum()) == 2
    # padding: rows >= N zero, k >= K zero; padded scale slots hold 127
    q2 = np.full((1, N, K), 0x11, np.uint8)
    qp2, sp2 = oracle_mod.pack(q2, s, 1, N, K)
    assert int((qp2 == 0x11).sum()) == N * K


@pytest.mark.parametrize("batch,N,K", [(1, 256, 128), (2, 300, 320), (3, 17, 96), (1, 512, 768)])
def test_pack_unpack_round_trip(oracle_mod, batch, N, K):
    rng = np.random.default_rng(batch * N + K)
    q = rng.integers(0, 256, (batch, N, K)).astype(np.uint8)
    s = rng.integers(0, 256, (batch, N, K // 32)).astype(np.uint8)
    qp, sp = oracle_mod.pack(q, s, batch, N, K)
    q2, s2 = oracle_mod.unpack(qp, sp, batch, N, K)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
