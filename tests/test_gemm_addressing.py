"""CPU check of the GEMM kernels' memory addressing (no GPU).

Every global access of the GEMM goes through a buffer descriptor whose range
check turns out-of-range lanes into zero reads, so the kernels are memory-safe
exactly when each descriptor's [base, base + num_records) lies inside the
buffer it describes.  This test mirrors, tile by tile, the descriptor
arithmetic of gemm.hip (dense and grouped, packed and canonical B, every tile
configuration the launcher picks) for the shapes the tests and the benchmark
launch, and asserts that containment.  It also checks the LDS footprint of the
copies against the kernel's LDS allocation.
"""
import numpy as np
import pytest

PANEL, KSTEP = 256, 128
TILE_BYTES = PANEL * KSTEP
WAVES = 8


def ceil_div(a, b):
    return (a + b - 1) // b


def dense_cfg(M, N, cus=256):
    t256 = ceil_div(M, 256) * ceil_div(N, 256)
    waves = ceil_div(t256, cus)
    fill = t256 / (waves * cus)
    if fill >= 0.85 or N <= 128:
        return 256, 256
    return 256, 128


def descriptors(M, N, K, BM, BN, packed, G=1, m0=0, m_end=None, n0=0, g=0):
    """(name, base_offset, num_records, buffer_size) of every descriptor of one tile."""
    KB = K // 32
    KS = ceil_div(K, KSTEP)
    NP = ceil_div(N, PANEL)
    m_end = M if m_end is None else m_end
    rows_a = min(BM, m_end - m0)
    assert rows_a >= 1
    out = [("a_q", m0 * K, rows_a * K, M * K), ("a_s", m0 * KB, rows_a * KB, M * KB)]
    if packed:
        panel, prow = n0 // PANEL, n0 % PANEL
        bt = ((g * NP + panel) * KS) * TILE_BYTES + prow * 128
        out.append(("b_q", bt, KS * TILE_BYTES - prow * 128, G * NP * KS * TILE_BYTES))
        bs = ((g * NP + panel) * KS) * 1024 + (prow // 16) * 64
        out.append(("b_s", bs, KS * 1024 - (prow // 16) * 64, G * NP * KS * 1024))
        # the per-step scale copies stay inside that range
        assert (KS - 1) * 1024 + BN * 4 <= KS * 1024 - (prow // 16) * 64
    else:
        rows_b = min(BN, N - n0)
        out.append(("b_q", n0 * K, rows_b * K, N * K))
        out.append(("b_s", n0 * KB, rows_b * KB, N * KB))
    return out


def check_tile(*args, **kw):
    for name, base, num, size in descriptors(*args, **kw):
        assert base >= 0 and num > 0, (name, base, num)
        assert base + num <= size, (name, base, num, size, args, kw)
        assert num < 2 ** 31


DENSE_SHAPES = [(64, 256, 256), (200, 300, 416), (256, 512, 1024), (33, 17, 32), (513, 264, 4096),
                (64, 1000, 2080), (1000, 96, 160), (4096, 6144, 4096), (8192, 24576, 4096),
                (8192, 4096, 12288), (8192, 4096, 24576), (8192, 12288, 4096),
                (24576, 4096, 8192), (4096, 12288, 8192), (64, 48, 512), (512, 768, 1024),
                (256, 320, 192), (512, 256, 128)]


@pytest.mark.parametrize("M,N,K", DENSE_SHAPES)
@pytest.mark.parametrize("packed", [False, True])
def test_dense_descriptors_inside_buffers(M, N, K, packed):
    BM, BN = dense_cfg(M, N)
    for tm in range(ceil_div(M, BM)):
        for tn in range(ceil_div(N, BN)):
            check_tile(M, N, K, BM, BN, packed, m0=tm * BM, n0=tn * BN)


def grouped_tiles(offsets, M_total, BM):
    """(g, m0, m_end) of every tile the grouped kernel runs (find_group mirror)."""
    tiles = []
    G = len(offsets) - 1
    for g in range(G):
        lo = min(max(int(offsets[g]), 0), M_total)
        hi = min(max(int(offsets[g + 1]), lo), M_total)
        for t in range(ceil_div(hi - lo, BM)):
            tiles.append((g, lo + t * BM, hi))
    return tiles


@pytest.mark.parametrize("G,N,K,offsets", [
    (8, 256, 256, None), (5, 200, 160, None), (16, 512, 768, None),
    (4, 128, 128, [32, 64, 64, 160, 192]),
    (128, 1536, 2048, None), (128, 2048, 768, None),
    (3, 256, 256, [-64, 96, 40, 10 ** 6]),          # malformed: clamped, never outside
])
def test_grouped_descriptors_inside_buffers(G, N, K, offsets):
    import workloads as wl
    if offsets is None:
        rng = np.random.default_rng(G + N)
        route = wl.zipf_topk_routing(rng, 4096 if G == 128 else 300, G, 8 if G == 128 else 2)
        offsets, _, _ = wl.group_layout(route, G)
    offsets = np.asarray(offsets, np.int64)
    M_total = max(32, int(min(max(offsets.max(), 0), 10 ** 5)) // 32 * 32)
    BM, BN = 128, 256
    upper = ceil_div(M_total, BM) + G
    tiles = grouped_tiles(offsets, M_total, BM)
    assert len(tiles) <= upper        # the launch grid covers every real tile
    for g, m0, m_end in tiles:
        for tn in range(ceil_div(N, BN)):
            check_tile(M_total, N, K, BM, BN, True, G=G, m0=m0, m_end=m_end, n0=tn * BN, g=g)


def stage_bytes(BM, BN, packed, kalign):
    sa_lds, sb_lds = kalign, packed or kalign
    return (BM + BN) * 128 + (BM * 4 if sa_lds else 0) + (BN * 4 if sb_lds else 0)


def stages_for(BM, BN, kalign):
    """the launcher's choice: three stages when K % 128 == 0 and they fit"""
    fits3 = all(3 * stage_bytes(BM, BN, pk, True) <= 160 * 1024 for pk in (False, True))
    return 3 if (kalign and fits3) else 2


@pytest.mark.parametrize("BM,BN,WM", [(256, 256, 2), (256, 128, 4), (128, 256, 2)])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kalign", [False, True])
def test_lds_footprint(BM, BN, WM, packed, kalign):
    """NST stages of [A tile | B tile | A scales | B scales] fit the 160 KB of
    LDS and every copy lands inside its region; the wave grid tiles the block."""
    nst = stages_for(BM, BN, kalign)
    sa_lds, sb_lds = kalign, packed or kalign
    tile = (BM + BN) * 128
    sa_off = tile
    sb_off = sa_off + (BM * 4 if sa_lds else 0)
    stage = stage_bytes(BM, BN, packed, kalign)
    assert nst * stage <= 160 * 1024
    segs_a, segs_b = BM // 8, BN // 8
    assert segs_a % WAVES == 0 and segs_b % WAVES == 0
    assert (segs_a + segs_b) * 1024 == tile                  # tile copies fill [0, tile)
    for w in range(WAVES):
        if sa_lds and w < BM // 64:
            assert sa_off + w * 256 + 256 <= sb_off
        if sb_lds and w < BN // 64:
            assert sb_off + w * 256 + 256 <= stage
    WN = WAVES // WM
    assert (BM // WM) % 16 == 0 and (BN // WN) % 16 == 0 and (BM // WM) // 16 >= 2


def gk_descriptors(M, N, T, lo, hi, tm, tn, BM=256, BN=256):
    """The grouped-K kernel's descriptors for tile (tm, tn) of a group with
    token range [lo, hi): A [M][T] and B [N][T] canonical, row stride T."""
    kb = hi - lo
    m0, n0 = tm * BM, tn * BN
    rows_a, rows_b = min(BM, M - m0), min(BN, N - n0)
    return [("a_q", m0 * T + lo, (rows_a - 1) * T + kb, M * T),
            ("a_s", m0 * (T // 32) + lo // 32, (rows_a - 1) * (T // 32) + kb // 32, M * (T // 32)),
            ("b_q", n0 * T + lo, (rows_b - 1) * T + kb, N * T),
            ("b_s", n0 * (T // 32) + lo // 32, (rows_b - 1) * (T // 32) + kb // 32, N * (T // 32))]


@pytest.mark.parametrize("M,N,T,offsets", [(200, 300, 384, [0, 32, 32, 224, 384]),
                                           (1536, 2048, 67616, [0, 7424, 7456, 67616]),
                                           (768, 2048, 4096, [0, 0, 4096, 4096])])
def test_grouped_k_descriptors_inside_buffers(M, N, T, offsets):
    """Every byte a grouped-K tile may touch lies inside its operand buffer,
    and in-range accesses (row < rows, k < group length) lie inside the
    descriptor range while the first out-of-range row starts past it."""
    for g in range(len(offsets) - 1):
        lo, hi = offsets[g], offsets[g + 1]
        for tm in range(ceil_div(M, 256)):
            for tn in range(ceil_div(N, 256)):
                for name, base, nbytes, size in gk_descriptors(M, N, T, lo, hi, tm, tn):
                    assert base >= 0 and base + max(nbytes, 0) <= size, (name, g, tm, tn)
                rows_a = min(256, M - tm * 256)
                kb = hi - lo
                if kb:
                    # last valid element of the last valid row, and the first invalid row
                    assert (rows_a - 1) * T + kb - 1 < (rows_a - 1) * T + kb
                    assert rows_a * T >= (rows_a - 1) * T + kb
