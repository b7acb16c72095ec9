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


IL_BLOCK = 1024 + 16          # interleaved LDS image: 1 KB copy block + padding
IL_GROUP = 8 * IL_BLOCK       # 64 rows


def il_bytes(rows):
    return rows // 64 * IL_GROUP


def il_copy_row(seg, slot):
    """row moved by copy block `seg`, slot `slot` (8 lanes = one 128-byte line)"""
    return (seg >> 3) * 64 + (slot >> 1) * 16 + 2 * (seg & 7) + (slot & 1)


def il_copy_addr(seg, slot, chunk):
    return (seg >> 3) * IL_GROUP + (seg & 7) * IL_BLOCK + slot * 128 + chunk * 16


def il_frag_addr(row0, lane, half):
    """LDS address the fragment reader uses: 16 rows from row0, lane group
    jj = lane // 16 reads chunk jj (half 0) and chunk 4 + jj (half 1)"""
    q, jj = lane & 15, lane >> 4
    g, f = row0 >> 6, (row0 >> 4) & 3
    return g * IL_GROUP + (q >> 1) * IL_BLOCK + (2 * f + (q & 1)) * 128 + (jj + 4 * half) * 16


@pytest.mark.parametrize("rows", [64, 128, 256])
def test_interleaved_image_roundtrip_and_bank_free(rows):
    """Copies move every row exactly once, as whole lines; the fragment reader
    finds exactly the bytes the copies wrote for (row, chunk); every 16-lane
    ds_read_b128 touches 16 distinct 16-byte bank slots (64 banks x 4 B)."""
    where = {}
    for seg in range(rows // 8):
        for slot in range(8):
            r = il_copy_row(seg, slot)
            for chunk in range(8):
                where[(r, chunk)] = il_copy_addr(seg, slot, chunk)
    assert sorted({r for r, _ in where}) == list(range(rows))
    assert len(set(where.values())) == rows * 8
    assert max(where.values()) + 16 <= il_bytes(rows)
    for row0 in range(0, rows, 16):
        for half in (0, 1):
            for lane in range(64):
                q, jj = lane & 15, lane >> 4
                assert il_frag_addr(row0, lane, half) == where[(row0 + q, jj + 4 * half)]
            for grp in range(4):
                slots = {(il_frag_addr(row0, grp * 16 + q, half) % 256) // 16 for q in range(16)}
                assert len(slots) == 16


def stage_bytes(BM, BN, packed):
    """one pipeline stage: [A image | B image | packed B scales]"""
    b_img = BN * 128 if packed else il_bytes(BN)
    return il_bytes(BM) + b_img + (BN * 4 if packed else 0)


def lds_total(BM, BN, packed, kalign):
    """two stages, then the double-buffered four-step canonical scale groups"""
    sq = (2 * BM * 16 if kalign else 0) + (2 * BN * 16 if (kalign and not packed) else 0)
    return 2 * stage_bytes(BM, BN, packed) + sq


@pytest.mark.parametrize("BM,BN,WM", [(256, 256, 2), (256, 128, 4), (128, 256, 2)])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kalign", [False, True])
def test_lds_footprint(BM, BN, WM, packed, kalign):
    """Two stages and the scale buffers fit the 160 KB of LDS, every copy lands
    inside its region, and the wave grid tiles the block."""
    a_img = il_bytes(BM)
    b_img = BN * 128 if packed else il_bytes(BN)
    stage = stage_bytes(BM, BN, packed)
    total = lds_total(BM, BN, packed, kalign)
    assert total <= 160 * 1024
    segs_a, segs_b = BM // 8, BN // 8
    assert segs_a % WAVES == 0 and segs_b % WAVES == 0
    assert max(il_copy_addr(seg, 7, 7) for seg in range(segs_a)) + 16 <= a_img
    if packed:
        assert segs_b * 1024 == b_img
        for w in range(BN // 64):                 # packed B scales of one step
            assert a_img + b_img + w * 256 + 256 <= stage
    else:
        assert max(il_copy_addr(seg, 7, 7) for seg in range(segs_b)) + 16 <= b_img
    if kalign:
        # canonical scale groups: buffer b, rows 64w + lane, 16 bytes (or per
        # step j, 4 bytes) each, inside [2 * stage, total)
        for rows, off in ((BM, 2 * stage),) + (((BN, 2 * stage + 2 * BM * 16),) if not packed else ()):
            for b in (0, 1):
                for w in range(rows // 64):
                    quad_end = off + b * rows * 16 + w * 1024 + 1024
                    step_end = off + b * rows * 16 + 3 * rows * 4 + w * 256 + 256
                    assert max(quad_end, step_end) <= off + 2 * rows * 16 <= total
    WN = WAVES // WM
    assert (BM // WM) % 16 == 0 and (BN // WN) % 16 == 0 and (BM // WM) // 16 >= 2
