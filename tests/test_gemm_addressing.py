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


def dense_tiling(M, N, cus=256):
    """Mirror of the launcher's dense tiling: (big_cols, small_cols) tile
    columns of 256x256 tiles, then of 256x128 tiles, minimising the estimated
    rounds of tiles (a 256x128 tile costs 0.66 of a 256x256 one)."""
    small = 0.66
    tm, tn_big, tn_small = ceil_div(M, 256), ceil_div(N, 256), ceil_div(N, 128)
    best, best_t = (tn_big, 0), ceil_div(tm * tn_big, cus)
    if N <= 128:
        return best
    t = small * ceil_div(tm * tn_small, cus)
    if t < best_t:
        best, best_t = (0, tn_small), t
    rounds = 1
    while rounds * cus < tm * tn_big:
        cols = rounds * cus // tm
        while cols > 0 and (tm * cols) % 8:
            cols -= 1
        if 0 < cols < tn_big:
            rest = ceil_div(N - cols * 256, 128)
            t = ceil_div(tm * cols, cus) + small * ceil_div(tm * rest, cus)
            if t < best_t - 1e-9:
                best, best_t = (cols, rest), t
        rounds += 1
    return best


def dense_tiles(M, N):
    """(m0, n0, BM, BN) of every tile of a dense launch."""
    big, small = dense_tiling(M, N)
    out = []
    for tm in range(ceil_div(M, 256)):
        out += [(tm * 256, tn * 256, 256, 256) for tn in range(big)]
        out += [(tm * 256, big * 256 + tn * 128, 256, 128) for tn in range(small)]
    return out


def test_dense_tiling_covers_c_once():
    """Every column of C lies in exactly one tile column, the mixed launch's
    large-tile count is a multiple of 8, and the qkv layer takes the mixed form."""
    for M, N, K in DENSE_SHAPES + [(500, 32968, 160), (512, 32768, 256)]:
        big, small = dense_tiling(M, N)
        assert big * 256 + small * 128 >= N                      # every column covered
        if small:
            assert big * 256 + (small - 1) * 128 < N             # no empty small column
        else:
            assert (big - 1) * 256 < N                           # no empty large column
        if big and small:
            assert (ceil_div(M, 256) * big) % 8 == 0
    assert dense_tiling(4096, 6144) == (16, 16)
    assert dense_tiling(500, 32968) == (128, 2)
    assert dense_tiling(8192, 24576) == (96, 0)
    assert dense_tiling(1024, 6144) == (0, 48)


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


def packed_a_descriptors(M, K, m0):
    """The packed-A descriptors of a tile starting at row m0 (a multiple of 8):
    from panel m0 / 256 on, two panels where there are two (a grouped tile
    may run into the next panel), all their k-step tiles and scale tiles."""
    KS = ceil_div(K, KSTEP)
    MP = ceil_div(M, PANEL)
    pa = m0 // PANEL
    n = min(2, MP - pa)
    return [("a_q", pa * KS * TILE_BYTES, n * KS * TILE_BYTES, MP * KS * TILE_BYTES),
            ("a_s", pa * KS * 1024, n * KS * 1024, MP * KS * 1024)]


def apack_offsets(m0, m_end, K, ks):
    """Mirror of TileOps::apack_off / apack_scale_off: per 8-row segment the
    byte offset of lane 0 (None past the tile's rows), per 16-row atom the
    offset of its 64-byte scale record."""
    KS = ceil_div(K, KSTEP)
    r0, rows = m0 % PANEL, min(256, m_end - m0)
    segs = [None if s * 8 >= rows else ((r0 + s * 8) // 256 * KS + ks) * TILE_BYTES + (r0 + s * 8) % 256 * 128
            for s in range(32)]
    atoms = [None if a * 16 >= rows else ((r0 + a * 16) // 256 * KS + ks) * 1024 + (r0 + a * 16) % 256 // 16 * 64
             for a in range(16)]
    return segs, atoms


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (200, 300, 512), (1000, 96, 1024), (513, 264, 4096),
                                   (2048, 9216, 512), (512, 32768, 256), (4096, 6144, 4096),
                                   (8192, 24576, 4096), (8192, 4096, 12288)])
def test_packed_a_descriptors_inside_buffers(M, N, K):
    for m0, n0, BM, BN in dense_tiles(M, N):
        for name, base, num, size in packed_a_descriptors(M, K, m0) + \
                [d for d in descriptors(M, N, K, BM, BN, True, m0=m0, n0=n0) if d[0].startswith("b")]:
            assert base >= 0 and num > 0 and base + num <= size, (name, M, N, K, m0)
            assert num < 2 ** 31
        # every step's copies (32 KB tile, 1 KB of scales) stay inside the ranges
        KS = ceil_div(K, KSTEP)
        assert (KS - 1) * TILE_BYTES + BM * 128 <= KS * TILE_BYTES
        assert (KS - 1) * 1024 + BM * 4 <= KS * 1024


def check_tile(*args, **kw):
    for name, base, num, size in descriptors(*args, **kw):
        assert base >= 0 and num > 0, (name, base, num)
        assert base + num <= size, (name, base, num, size, args, kw)
        assert num < 2 ** 31


DENSE_SHAPES = [(64, 256, 256), (200, 300, 416), (256, 512, 1024), (33, 17, 32), (513, 264, 4096),
                (64, 1000, 2080), (1000, 96, 160), (4096, 6144, 4096), (8192, 24576, 4096),
                (8192, 4096, 12288), (8192, 4096, 24576), (8192, 12288, 4096),
                (24576, 4096, 8192), (4096, 12288, 8192), (64, 48, 512), (512, 768, 1024),
                (256, 320, 192), (512, 256, 128), (500, 32968, 160), (512, 32768, 256),
                (2048, 12288, 4096), (3072, 6144, 4096)]


@pytest.mark.parametrize("M,N,K", DENSE_SHAPES)
@pytest.mark.parametrize("packed", [False, True])
def test_dense_descriptors_inside_buffers(M, N, K, packed):
    for m0, n0, BM, BN in dense_tiles(M, N):
        check_tile(M, N, K, BM, BN, packed, m0=m0, n0=n0)


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
    BM, BN = (256 if M_total >= 256 * G else 128), 256     # the launcher's choice
    upper = ceil_div(M_total, BM) + G
    tiles = grouped_tiles(offsets, M_total, BM)
    assert len(tiles) <= upper        # the launch grid covers every real tile
    for g, m0, m_end in tiles:
        for tn in range(ceil_div(N, BN)):
            check_tile(M_total, N, K, BM, BN, True, G=G, m0=m0, m_end=m_end, n0=tn * BN, g=g)


def check_epilogue_stores(M, N, BM, BN, WM, m0, m_end, n0, es):
    """Mirror of store_tile_lds's buffer stores: each wave's descriptor starts
    at its first row of C and spans its rows below m_end; every store of a
    row below m_end lies inside it, every store of a row at or past m_end lies
    past it (dropped), and the descriptor lies inside C (M x N elements)."""
    WN = WAVES // WM
    WTM, WTN = BM // WM, BN // WN
    if not (n0 + BN <= N and (N * es) % 16 == 0):
        return                                  # the element-by-element path
    if WTM * N * es > 0xFFFFFFFF:
        return                                  # pointer stores (count not exact)
    lpr = WTN * es // 16
    for w in range(WAVES):
        row0, col0 = m0 + (w // WN) * WTM, n0 + (w % WN) * WTN
        rows_here = m_end - row0
        if rows_here <= 0:
            continue                            # range 0: every store dropped
        base = (row0 * N + col0) * es
        rng = (min(rows_here, WTM) - 1) * N * es + WTN * es
        assert 0 <= base and base + rng <= M * N * es, (M, N, m0, m_end, n0, w)
        # offsets grow with the row and the lane: the extreme stores decide
        last = min(rows_here, WTM) - 1                 # last row below m_end
        assert last * N * es + (lpr - 1) * 16 + 16 <= rng
        assert (WTM - 1) * N * es + (lpr - 1) * 16 < 2 ** 32
        if rows_here < WTM:                            # first row at m_end: dropped
            assert rows_here * N * es >= rng


@pytest.mark.parametrize("M,N,K", DENSE_SHAPES[:12])
@pytest.mark.parametrize("es", [2, 4])
def test_epilogue_store_descriptors(M, N, K, es):
    for m0, n0, BM, BN in dense_tiles(M, N):
        check_epilogue_stores(M, N, BM, BN, 2 if BN == 256 else 4, m0, M, n0, es)


def test_epilogue_store_descriptors_grouped():
    import workloads as wl
    rng = np.random.default_rng(7)
    route = wl.zipf_topk_routing(rng, 4096, 128, 8)
    offsets, _, _ = wl.group_layout(route, 128)
    M_total = int(offsets[-1])
    for N in (1536, 2048):
        for g, m0, m_end in grouped_tiles(offsets, M_total, 256):
            for tn in range(ceil_div(N, 256)):
                check_epilogue_stores(M_total, N, 256, 256, 2, m0, m_end, tn * 256, 2)


def stage_bytes(BM, BN, packed, kalign):
    sa_lds, sb_lds = kalign, packed or kalign
    return (BM + BN) * 128 + (BM * 4 if sa_lds else 0) + (BN * 4 if sb_lds else 0)


def stages_for(BM, BN, kalign, grouped):
    """the launcher's choice: three stages for grouped launches when K % 128 == 0
    and they fit, else two"""
    fits3 = all(3 * stage_bytes(BM, BN, pk, True) <= 160 * 1024 for pk in (False, True))
    return 3 if (grouped and kalign and fits3) else 2


@pytest.mark.parametrize("BM,BN,WM,grouped", [(256, 256, 2, False), (256, 128, 4, False), (128, 256, 2, True),
                                               (256, 256, 2, True)])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kalign", [False, True])
def test_lds_footprint(BM, BN, WM, grouped, packed, kalign):
    """NST stages of [A tile | B tile | A scales | B scales] fit the 160 KB of
    LDS and every copy lands inside its region; the wave grid tiles the block.
    (The mixed dense launch allocates two stages of its larger tile.)"""
    nst = stages_for(BM, BN, kalign, grouped)
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


CHUNK_STEPS = 8


def check_chunk_copies(M, K, tiles):
    """tiles: (r0, r_end) of 256-row operand tiles over an operand of M rows"""
    KB, KS = K // 32, ceil_div(K, KSTEP)
    assert K % 512 == 0 and KB % 16 == 0
    chunks = ceil_div(KS, CHUNK_STEPS)
    for m0, m_end in tiles:
        rows_a = min(256, m_end - m0)
        base, num = m0 * KB, (rows_a - 1) * KB + KB
        assert base + num <= M * KB
        for w in range(WAVES):
            for lane in range(64):
                row = 32 * w + lane // 2
                h = (lane % 2) ^ (row // 8 % 2)
                for c in range(chunks):
                    off = row * KB + 32 * c + 16 * h
                    inside = off + 16 <= num
                    assert inside or off >= num, (M, K, m0, row, c)
                    if row < rows_a and 32 * c + 16 * h < KB:
                        assert inside                      # real scales arrive


def test_chunked_a_scale_copies_grouped():
    """The grouped GEMM's 256-row tiles (groups averaging 256 rows or more)
    take the same chunked A-scale copies when K % 512 == 0."""
    import workloads as wl
    rng = np.random.default_rng(7)
    for G, K, tokens in ((128, 2048, 8192), (16, 512, 2048)):
        route = wl.zipf_topk_routing(rng, tokens, G, 8)
        offsets, _, _ = wl.group_layout(route, G)
        M_total = int(offsets[-1])
        assert M_total >= 256 * G                   # the launcher takes 256-row tiles
        tiles = [(m0, m_end) for g, m0, m_end in grouped_tiles(offsets, M_total, 256)]
        check_chunk_copies(M_total, K, tiles)


@pytest.mark.parametrize("M,N,K", [s for s in DENSE_SHAPES if s[2] % 512 == 0] + [(300, 520, 1536), (77, 256, 512)])
def test_chunked_a_scale_copies(M, N, K):
    """Dense launches with K % 512 == 0 copy each tile's A scales in chunks of
    8 k-steps: wave w, lane l copies the 16 bytes at offset
    row * KB + 32c + 16 ((l % 2) ^ (row // 8 % 2)) of the tile's A-scale
    descriptor, row = 32w + l // 2.  Every piece must be wholly inside the descriptor's range
    (and so inside a_s) or wholly past it (read as zero, never partly), and
    the pieces that carry scales of real k-steps must be inside.  Mirrors
    gemm.hip's chunked A-scale path; also checks the LDS budget of the
    two chunk buffers beside the two stages."""
    tiles = dense_tiles(M, N)
    check_chunk_copies(M, K, [(m0, M) for m0, n0, BM, BN in tiles if BM == 256])
    # canonical B: the 256-row B tiles' scales are chunked the same way
    check_chunk_copies(N, K, [(n0, N) for m0, n0, BM, BN in tiles if BN == 256])
    # LDS: two stages without per-step A scales plus two 8 KB chunk buffers,
    # and (canonical B, 256-row B tiles) without per-step B scales plus two more
    for BM, BN, packed in ((256, 256, True), (256, 256, False), (256, 128, True), (256, 128, False)):
        sbc = not packed and BN == 256
        stage = (BM + BN) * 128 + (0 if sbc else BN * 4)
        big = (256 + 256) * 128 + (0 if not packed else 256 * 4)
        chunks = 2 * BM * 32 + (2 * 256 * 32 if not packed else 0)
        assert 2 * max(stage, big) + chunks <= 160 * 1024


def test_pair_kernel_lds_regions():
    """The paired launch (a 256x256 tile, then a 256x128 tile, per
    workgroup): before the first tile's epilogue, the second tile's step-0
    copies and scale chunk 0 go into the stage and chunk buffer the first
    tile's last step did not read, and the epilogue stages C only in the
    other stage; every region stays inside the allocation.  Mirrors
    gemm_pair_kernel's choice of F = KS % 2 and Lc = ((KS - 1) / 8) % 2."""
    SB = (256 + 256) * 128 + 256 * 4            # large-tile stage (packed B scales, chunked A)
    SS = (256 + 128) * 128 + 128 * 4            # small-tile stage
    CHUNK = 256 * 32
    total = 2 * SB + 2 * CHUNK
    assert total <= 160 * 1024 and SS <= SB
    for KS in range(1, 50):
        last_stage = (KS - 1) % 2
        last_chunk = ((KS - 1) // 8) % 2
        F, Lc = KS % 2, ((KS - 1) // 8) % 2
        assert F != last_stage and Lc == last_chunk
        small0 = (F * SB, F * SB + SS)                       # second tile's step 0
        epi = ((1 - F) * SB, (1 - F) * SB + SB)              # first tile's C staging
        chunk0 = (2 * SB + (1 - Lc) * CHUNK, 2 * SB + (2 - Lc) * CHUNK)
        in_use = [(last_stage * SB, last_stage * SB + SB), (2 * SB + Lc * CHUNK, 2 * SB + (Lc + 1) * CHUNK)]
        for a, b in (small0, chunk0):
            assert 0 <= a < b <= total
            for c, d in in_use:                               # nothing the last step reads
                assert b <= c or a >= d
            assert b <= epi[0] or a >= epi[1]                 # nor the staging area
        # C staging of the 256x256 tile fits one stage: 8 waves x 32 rows x (64 x 2 + 16) B
        assert 8 * 32 * (64 * 2 + 16) <= SB and 8 * 16 * (64 * 4 + 16) <= SB


@pytest.mark.parametrize("n", [1, 7, 8, 255, 256, 257, 1000, 3091])
@pytest.mark.parametrize("grid", [256, 80])
def test_grouped_persistent_tile_assignment(n, grid):
    """The persistent grouped launch: XCD x = workgroup % 8 owns tiles
    [n x / 8, n (x+1) / 8), its workgroups j = workgroup / 8 (nj of them)
    take lo + j, lo + j + nj, ...  Every tile exactly once."""
    seen = []
    for b in range(grid):
        x, j = b % 8, b // 8
        nj = (grid - x + 7) // 8
        lo, hi = n * x // 8, n * (x + 1) // 8
        seen += list(range(lo + j, hi, nj))
    assert sorted(seen) == list(range(n))


def test_grouped_persistent_lds_handover():
    """Between two tiles the persistent grouped launch issues the next tile's
    step 0 into the stage the finished tile's last step did not read and its
    scale chunk 0 into the chunk buffer that step did not read; C is staged
    in the other stage.  Mirrors st_free / c_free over tile sequences."""
    for sac in (False, True):
        SB = (256 + 256) * 128 + (0 if sac else 256 * 4) + 256 * 4
        CHUNK = 256 * 32
        total = 2 * SB + (2 * CHUNK if sac else 0)
        assert total <= 160 * 1024
        for KS in range(1, 40):
            st, ch_par = [0, SB], 0
            for _ in range(5):                                  # five tiles in a row
                last_stage = st[(KS - 1) % 2]
                last_chunk = ((KS - 1) // 8 + ch_par) % 2
                st_free, c_free = st[KS % 2], 1 - last_chunk
                assert st_free != last_stage and c_free != last_chunk
                assert st_free + SB <= 2 * SB and last_stage + SB <= 2 * SB
                # C staging (8 waves x 32 rows x 144 B) fits the busy stage
                assert 8 * 32 * (64 * 2 + 16) <= SB and 8 * 16 * (64 * 4 + 16) <= SB
                st, ch_par = [st_free, last_stage], c_free


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


def splitk_plan(M, N, K, cus=256):
    """Mirror of the split-K plan: (splits, k-steps per slice); 256x128 tiles."""
    tiles = ceil_div(M, 256) * ceil_div(N, 128)
    ks = ceil_div(K, KSTEP)
    if tiles * 2 > cus or ks < 8:
        return 1, ks
    s = min(cus // tiles, ks // 4)
    if s < 2:
        return 1, ks
    steps = ceil_div(ks, s)
    return ceil_div(ks, steps), steps


SPLITK_SHAPES = [(64, 256, 1024), (200, 300, 2080), (512, 6144, 4096), (1000, 96, 4128), (32, 4096, 12288),
                 (512, 4096, 4096), (256, 24576, 4096)]


@pytest.mark.parametrize("M,N,K", SPLITK_SHAPES)
@pytest.mark.parametrize("packed", [False, True])
def test_splitk_slices_cover_k_and_stay_inside(M, N, K, packed):
    """Every slice is non-empty, the slices tile [0, K) exactly, the grid fits
    one round, and every descriptor of every (slice, tile) -- A from its
    slice's first column, packed B from its slice's first k-step -- lies
    inside its buffer."""
    splits, steps = splitk_plan(M, N, K)
    KB, KS, NP = K // 32, ceil_div(K, KSTEP), ceil_div(N, PANEL)
    bounds = [(s * steps * KSTEP, min(steps * KSTEP, K - s * steps * KSTEP)) for s in range(splits)]
    assert all(kb > 0 for _, kb in bounds) and bounds[0][0] == 0
    assert sum(kb for _, kb in bounds) == K
    assert all(k0 % KSTEP == 0 for k0, _ in bounds)
    if splits > 1:
        assert ceil_div(M, 256) * ceil_div(N, 128) * splits <= 256
    for k0, kb in bounds:
        s0 = k0 // KSTEP
        for tm in range(ceil_div(M, 256)):
            m0 = tm * 256
            rows_a = min(256, M - m0)
            assert m0 * K + k0 + (rows_a - 1) * K + kb <= M * K
            assert m0 * KB + k0 // 32 + (rows_a - 1) * KB + kb // 32 <= M * KB
            for tn in range(ceil_div(N, 128)):
                n0 = tn * 128
                if packed:
                    panel, prow = n0 // PANEL, n0 % PANEL
                    base = (panel * KS + s0) * TILE_BYTES + prow * 128
                    assert base + (KS - s0) * TILE_BYTES - prow * 128 <= NP * KS * TILE_BYTES
                    sbase = (panel * KS + s0) * 1024 + (prow // 16) * 64
                    assert sbase + (KS - s0) * 1024 - (prow // 16) * 64 <= NP * KS * 1024
                else:
                    rows_b = min(128, N - n0)
                    assert n0 * K + k0 + (rows_b - 1) * K + kb <= N * K


def xcd_contiguous_tile(wg, nwg):
    q, r, x = nwg // 8, nwg % 8, wg % 8
    return x * q + min(x, r) + wg // 8


@pytest.mark.parametrize("shapes", [[(1, 256, 128)], [(1, 6144, 4096), (1, 4096, 4096), (1, 24576, 4096),
                                                       (1, 4096, 12288)],
                                    [(3, 17, 96), (1, 1, 32), (2, 300, 320)] * 10 + [(1, 513, 4160)]])
def test_packed_many_job_select(shapes):
    """CPU mirror of quantize_packed_kernel's job lookup: every workgroup of the
    launch lands on exactly one tile of exactly one weight, inside that
    weight's tile range, and every tile of every weight is taken once."""
    JMAX = 32
    assert len(shapes) <= JMAX
    tile_end, tot = [], 0
    for batch, N, K in shapes:
        tot += batch * ceil_div(N, 256) * ceil_div(K, 128)
        tile_end.append(tot)
    count = len(shapes)
    tile_end += [0] * (JMAX - count)               # unused table slots are zero
    seen = [set() for _ in shapes]
    for wg in range(tot):
        tidx = xcd_contiguous_tile(wg, tot)
        assert 0 <= tidx < tot
        j = 0
        for i in range(JMAX - 1):
            if i < count - 1 and tidx >= tile_end[i]:
                j = i + 1
        start = tile_end[j - 1] if j else 0
        local = tidx - start
        batch, N, K = shapes[j]
        assert 0 <= local < batch * ceil_div(N, 256) * ceil_div(K, 128)
        assert local not in seen[j]
        seen[j].add(local)
    for (batch, N, K), s in zip(shapes, seen):
        assert len(s) == batch * ceil_div(N, 256) * ceil_div(K, 128)


@pytest.mark.parametrize("shapes", [[(4096, 4096), (6144, 4096)], [(1, 32), (3, 96), (5, 4160), (64, 64)],
                                    [(7, 2048), (1, 32)] * 4])
def test_quantize_many_step_walk(shapes):
    """CPU mirror of quantize_axis1_many_kernel's walk: the waves of the launch
    visit every wave-step once; each step's tensor and local block range come
    from the running step totals; the blocks a step writes (block < nblocks
    of its tensor) cover every block of every tensor exactly once."""
    JMAX = 8
    assert len(shapes) <= JMAX
    nblocks = [r * c // 32 for r, c in shapes]
    step_end, tot = [], 0
    for nb in nblocks:
        tot += -(-nb // 64)
        step_end.append(tot)
    count = len(shapes)
    step_end += [0] * (JMAX - count)
    cus = 256
    grid = max(1, min(-(-tot // 4), cus * 32 // 4))
    nwaves = grid * 4
    covered = [np.zeros(nb, np.int32) for nb in nblocks]
    visited = np.zeros(tot, np.int32)
    for wave in range(nwaves):
        step = wave
        while step < tot:
            j = 0
            for i in range(JMAX - 1):
                if i < count - 1 and step >= step_end[i]:
                    j = i + 1
            local = step - (step_end[j - 1] if j else 0)
            assert 0 <= local < -(-nblocks[j] // 64)
            visited[step] += 1
            for lane in range(64):
                blk = local * 64 + lane
                if blk < nblocks[j]:
                    covered[j][blk] += 1
            step += nwaves
    assert np.all(visited == 1)
    for c in covered:
        assert np.all(c == 1)


@pytest.mark.parametrize("batch,rows,cols", [(1, 128, 256), (1, 96, 40), (3, 64, 296), (2, 320, 520),
                                             (1, 32, 8)])
def test_quantize_packed_axis0_writes_every_byte_once(batch, rows, cols):
    """CPU mirror of quantize_axis0_packed_kernel's stores: over the tile list
    (batch x k-steps x two halves per panel) every 16-byte code chunk and every
    scale word of the packed buffers is written exactly once, inside them."""
    KS, NP = ceil_div(rows, 128), ceil_div(cols, 256)
    q_chunks = np.zeros(batch * NP * KS * 256 * 8, np.int32)     # 16-byte chunks of q_packed
    s_words = np.zeros(batch * NP * KS * 256, np.int32)          # 4-byte words of scales_packed
    ntiles = batch * KS * 2 * NP
    for idx in range(ntiles):
        per = KS * 2 * NP
        b, t = idx // per, idx % per
        R0, C0 = (t // (2 * NP)) * 128, (t % (2 * NP)) * 128
        ks, h = R0 // 128, (C0 // 128) & 1
        tile_lin = (b * NP + C0 // 256) * KS + ks
        base = tile_lin * 256 * 128 + h * 128 * 128
        for th in range(256):
            for i in range(4):
                col, j = i * 32 + (th >> 3), th & 7
                off = base + col * 128 + ((j ^ (col & 7)) << 4)
                assert off % 16 == 0
                q_chunks[off // 16] += 1
            if th < 128:
                s_words[tile_lin * 256 + h * 128 + th] += 1
    assert np.all(q_chunks == 1) and np.all(s_words == 1)


@pytest.mark.parametrize("rows,cols", [(1, 32), (17, 4128), (300, 320), (513, 1056), (256, 128), (4096, 4096)])
def test_quantize_many_packed_steps_write_every_byte_once(rows, cols):
    """Mirror of the list quantizer's packed steps (mxfp8_quantize_many_layouts):
    step = (16-row atom, k-step); lane l holds half l % 2 of block (l / 2) % 4
    of row 8h + l / 8 in sub-step h.  Every byte of the packed codes and
    scales is written exactly once; each code chunk lands at its row's slot
    c ^ (row % 8); each scale byte comes from the lane that holds that row's
    block (the shuffle source)."""
    KS = ceil_div(cols, KSTEP)
    atoms = ceil_div(rows, PANEL) * 16
    st = np.arange(atoms * KS)
    atom, ks = st // KS, st % KS
    lane = np.arange(64)
    bl, half = lane >> 1, lane & 1
    i, kb4 = bl >> 2, bl & 3
    tile_lin = (atom // 16) * KS + ks
    qcount = np.zeros(ceil_div(rows, PANEL) * KS * TILE_BYTES // 16, np.int64)
    for h in (0, 1):
        rp = (atom[:, None] % 16) * 16 + h * 8 + i[None, :]
        c = kb4 * 2 + half
        off = tile_lin[:, None] * TILE_BYTES + rp * 128 + ((c[None, :] ^ (rp & 7)) << 4)
        assert np.all(off % 16 == 0)
        np.add.at(qcount, (off // 16).ravel(), 1)
        # the chunk holds K bytes 32 kb4 + 16 half .. +15 of row rp: chunk c
        assert np.all(((kb4 * 32 + half * 16) // 16) == c)
    assert np.all(qcount == 1)
    soff = tile_lin[:, None] * 1024 + (atom[:, None] % 16) * 64 + lane[None, :]
    scount = np.bincount(soff.ravel(), minlength=ceil_div(rows, PANEL) * KS * 1024)
    assert np.all(scount == 1)
    # scale byte l: row l % 16 (sub-step row // 8), block l // 16; its code is
    # held by lane 2 * (4 * (row % 8) + block), which owns that row and block
    rr = lane & 15
    src = 2 * ((rr & 7) * 4 + (lane >> 4))
    assert np.all(((src >> 1) >> 2) == (rr & 7)) and np.all(((src >> 1) & 3) == (lane >> 4))



# ---- gemm_ws_kernel (packed A and B, 256x128 tiles, copying and computing waves)

WS_STAGE = 256 * 128 + 128 * 128 + 256 * 4 + 128 * 4       # A rows | B rows | A scales | B scales


def grouped_order(L, tiles_m, tiles_n, group_m=4):
    per = group_m * tiles_n
    gid, inn = L // per, L % per
    first = gid * group_m
    gsz = min(tiles_m - first, group_m)
    return first + inn % gsz, inn // gsz


def ws_tiles(wg, nwg, T):
    """Mirror of ws_tiles: (first, stride, count) of workgroup wg."""
    q, r, x, j = nwg // 8, nwg % 8, wg % 8, wg // 8
    nx = q + (1 if x < r else 0)
    before = x * q + min(x, r)
    lo, hi = T * before // nwg, T * (before + nx) // nwg
    first = lo + j
    return first, nx, (hi - first + nx - 1) // nx if first < hi else 0


@pytest.mark.parametrize("T", [1, 3, 7, 8, 9, 255, 256, 257, 768, 1000, 6144])
def test_ws_tile_assignment(T):
    """Every tile exactly once, for grids of min(T, CUs) workgroups (also
    grids smaller than 8, which leave XCDs without workgroups)."""
    for cus in (256, 80, 304):
        nwg = min(T, cus)
        seen = []
        for wg in range(nwg):
            first, stride, count = ws_tiles(wg, nwg, T)
            seen += [first + i * stride for i in range(count)]
        assert sorted(seen) == list(range(T)), (T, cus)
        counts = [ws_tiles(wg, nwg, T)[2] for wg in range(nwg)]
        assert max(counts) - min(counts) <= 2, (T, cus)


WS_SHAPES = [(64, 256, 256), (200, 300, 512), (1000, 96, 1024), (513, 264, 4096), (2048, 9216, 512),
             (512, 32768, 256), (4096, 6144, 4096), (8192, 24576, 4096), (8192, 4096, 12288), (33, 4, 128),
             (300, 132, 384)]


@pytest.mark.parametrize("M,N,K", WS_SHAPES)
def test_ws_copies_inside_buffers(M, N, K):
    """The copying waves' descriptors (A panel, B half panel and their scale
    tiles from k-step 0) lie inside the packed buffers, every copy of every
    step lies inside its descriptor, and every LDS target inside its stage."""
    assert 3 * WS_STAGE + 4 * 16 * (64 * 2 + 16) <= 160 * 1024     # ring + the computing waves' band buffers
    KS, MP, NP = ceil_div(K, KSTEP), ceil_div(M, PANEL), ceil_div(N, PANEL)
    tiles_m, tiles_n = ceil_div(M, 256), ceil_div(N, 128)
    for L in range(tiles_m * tiles_n):
        tm, tn = grouped_order(L, tiles_m, tiles_n)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        pa, pb, prow = tm, tn * 128 // PANEL, tn * 128 % PANEL
        descs = [(pa * KS * TILE_BYTES, KS * TILE_BYTES, MP * KS * TILE_BYTES),
                 (pa * KS * 1024, KS * 1024, MP * KS * 1024),
                 (pb * KS * TILE_BYTES + prow * 128, KS * TILE_BYTES - prow * 128, NP * KS * TILE_BYTES),
                 (pb * KS * 1024 + prow // 16 * 64, KS * 1024 - prow // 16 * 64, NP * KS * 1024)]
        for base, num, size in descs:
            assert base >= 0 and 0 < num < 2 ** 32 and base + num <= size, (M, N, K, tm, tn)
        last = (KS - 1) * TILE_BYTES
        for pw in range(4):
            a_end = max(last + (i * 4 + pw) * 1024 + 63 * 16 + 16 for i in range(8))
            b_end = max(last + (i * 4 + pw) * 1024 + 63 * 16 + 16 for i in range(4))
            s_end = (KS - 1) * 1024 + pw * 256 + 63 * 4 + 4
            assert a_end <= descs[0][1] and b_end <= descs[2][1] and s_end <= descs[1][1]
            if pw < 2:
                assert s_end <= descs[3][1]
            # LDS targets: A segments, B segments, scale dwords, inside one stage
            assert max((i * 4 + pw) * 1024 + 1024 for i in range(8)) <= 256 * 128
            assert 256 * 128 + max((i * 4 + pw) * 1024 + 1024 for i in range(4)) <= 256 * 128 + 128 * 128
            assert 256 * 128 + 128 * 128 + pw * 256 + 256 <= 256 * 128 + 128 * 128 + 1024
        assert 256 * 128 + 128 * 128 + 1024 + 2 * 256 == WS_STAGE


@pytest.mark.parametrize("M,N", [(64, 256), (200, 304), (1000, 96), (513, 264), (33, 4), (300, 132),
                                 (256, 128), (4096, 6144), (40, 72)])
@pytest.mark.parametrize("es", [2, 4])
def test_ws_stores_cover_c_once(M, N, es):
    """Each computing wave's stores through a descriptor spanning its block
    of C (fp32: one 4-column piece per lane and 16x16 tile; bf16: 16-row
    bands, one 8-column piece per lane, eight lanes per row): every piece
    inside the range, every element of C written exactly once."""
    if N % (8 if es == 2 else 4):
        pytest.skip("the launcher takes this kernel only for N % 8 == 0 (bf16) or N % 4 == 0 (fp32)")
    tiles_m, tiles_n = ceil_div(M, 256), ceil_div(N, 128)
    hits = np.zeros(M * N, np.int32)
    lane = np.arange(64)
    for L in range(tiles_m * tiles_n):
        tm, tn = grouped_order(L, tiles_m, tiles_n)
        for w in range(4):
            wm, wn = w >> 1, w & 1
            row0, col0 = tm * 256 + wm * 128, tn * 128 + wn * 64
            rows_here, cols_here = M - row0, N - col0
            if rows_here <= 0 or cols_here <= 0:
                continue
            rh, chh = min(rows_here, 128), min(cols_here, 64)
            rng = ((rh - 1) * N + chh) * es
            base = (row0 * N + col0) * es
            assert base + rng <= M * N * es and rng < 2 ** 31
            g = lane >> 4
            if es == 2:        # 16-row bands through LDS: 8 lanes per 128-byte row, two stores per band
                pieces = [(h * 8 + (lane >> 3), (lane & 7) * 8, 8) for h in range(2)]
            else:              # 16 bytes per lane and 16x16 tile
                pieces = [(lane & 15, j * 16 + g * 4, 4) for j in range(4)]
            for i in range(8):
                for rb, cl, width in pieces:
                    r = i * 16 + rb
                    ok = (r < rh) & (cl < chh)
                    off = (r * N + cl) * es
                    assert np.all(off[ok] + width * es <= rng)
                    assert 0x80000000 >= rng
                    for c in range(width):
                        np.add.at(hits, (row0 + r[ok]) * N + col0 + cl[ok] + c, 1)
    assert np.all(hits == 1), (M, N)


def packed_tiling(M, N, es, cus=256):
    """Mirror of packed_tiling: 'ws' (256x128 tiles), 'half' (128x128) or
    'dense' (launch_gemm's tilings)."""
    tm, full = ceil_div(M, 256), ceil_div(M, 256) * ceil_div(N, 128)
    if N % (8 if es == 2 else 4) or 128 * N * es >= 2 ** 31 or full > 3 * cus:
        return "dense"
    t_full = ceil_div(full, cus)
    t_half = 0.67 * ceil_div(ceil_div(M, 128) * ceil_div(N, 128), cus)
    t_big = 1.5 * ceil_div(tm * ceil_div(N, 256), cus)
    if t_big < t_full - 1e-9 and t_big < t_half - 1e-9:
        return "dense"
    return "half" if t_half < t_full - 1e-9 else "ws"


def test_packed_tiling_choices():
    """The Qwen3-8B linears: 128-row tiles where 256-row ones leave most CUs
    idle, 256x256 tiles where 256x128 ones take one and a half rounds."""
    assert packed_tiling(512, 6144, 2) == "half" and packed_tiling(512, 4096, 2) == "half"
    assert packed_tiling(512, 24576, 2) == "dense" and packed_tiling(512, 4096, 2, cus=80) == "ws"
    assert packed_tiling(1024, 6144, 2) == "ws" and packed_tiling(4096, 6144, 2) == "ws"
    assert packed_tiling(8192, 24576, 2) == "dense" and packed_tiling(512, 6148, 2) == "dense"


@pytest.mark.parametrize("M,N,K", [(512, 6144, 4096), (512, 4096, 4096), (100, 264, 512), (384, 136, 256),
                                   (129, 8, 128), (640, 1024, 1024)])
@pytest.mark.parametrize("es", [2, 4])
def test_ws_half_tiles_copy_their_rows_and_store_once(M, N, K, es):
    """128-row tiles (tm: rows tm*128..+127, the upper or lower half of
    panel tm/2): the copying waves' four A segments per k-step bring exactly
    those rows into LDS rows 0..127 (each once, inside the panel's
    descriptor), waves 0 and 1 copy the half's eight scale atoms into LDS
    atoms 0..7 (waves 2 and 3 copy nothing: kOOB), and the computing waves of
    rows 0..127 write every element of C once."""
    if N % (8 if es == 2 else 4):
        pytest.skip("the launcher takes this kernel only for N % 8 == 0 (bf16) or N % 4 == 0 (fp32)")
    KS, MP = ceil_div(K, KSTEP), ceil_div(M, PANEL)
    tiles_m, tiles_n = ceil_div(M, 128), ceil_div(N, 128)
    lane = np.arange(64)
    hits = np.zeros(M * N, np.int32)
    for L in range(tiles_m * tiles_n):
        tm, tn = grouped_order(L, tiles_m, tiles_n)
        pa, a_m0 = tm // 2, (tm % 2) * 128
        assert pa < MP and pa * KS * TILE_BYTES + KS * TILE_BYTES <= MP * KS * TILE_BYTES
        for ks in (0, KS - 1):
            k0 = ks * TILE_BYTES
            rows = np.zeros(256, np.int32)
            for pw in range(4):
                for i in range(4):
                    seg = i * 4 + pw
                    off = k0 + a_m0 * 128 + seg * 1024 + lane * 16
                    assert off.max() + 16 <= KS * TILE_BYTES
                    lds = seg * 1024 + lane * 16
                    # a panel row's 128 bytes land on the tile row's 128 bytes
                    assert np.all((off - k0) // 128 - a_m0 == lds // 128) and np.all(off % 128 == lds % 128)
                    np.add.at(rows, (off - k0) // 128, 1)
                if pw < 2:
                    s_off = ks * 1024 + pw * 256 + lane * 4 + a_m0 * 4
                    assert s_off.max() + 4 <= KS * 1024
                    assert np.all(s_off // 64 - ks * 16 - a_m0 // 16 == (pw * 256 + lane * 4) // 64)
            want = np.zeros(256, np.int32)
            want[a_m0:a_m0 + 128] = 8           # 8 lanes (16 bytes each) per row
            assert np.array_equal(rows, want)
        row0, row_end = tm * 128, min(M, tm * 128 + 128)
        for wn in range(2):
            col0 = tn * 128 + wn * 64
            rh, chh = row_end - row0, min(N - col0, 64)
            if rh <= 0 or chh <= 0:
                continue
            rng = ((rh - 1) * N + chh) * es
            assert (row0 * N + col0) * es + rng <= M * N * es
            if es == 2:
                pieces = [(h * 8 + (lane >> 3), (lane & 7) * 8, 8) for h in range(2)]
            else:
                pieces = [(lane & 15, j * 16 + (lane >> 4) * 4, 4) for j in range(4)]
            for i in range(8):
                for rb, cl, width in pieces:
                    r = i * 16 + rb
                    ok = (r < rh) & (cl < chh)
                    assert np.all((r[ok] * N + cl[ok]) * es + width * es <= rng)
                    for c in range(width):
                        np.add.at(hits, (row0 + r[ok]) * N + col0 + cl[ok] + c, 1)
    assert np.all(hits == 1), (M, N)


@pytest.mark.parametrize("M,N,K", [(64, 256, 1024), (300, 4096, 4096), (512, 6144, 4096), (512, 4096, 12288),
                                   (32, 1000, 2048)])
def test_ws_split_units_cover_k_and_partials_stay_inside(M, N, K):
    """The split launch of gemm_ws_kernel: units u = (tile u % T, slice u / T)
    dealt like tiles; every unit has at least one k-step, each tile's slices
    tile [0, KS) exactly, and every partial store (the fp32 path, slice s at
    s * c_stride elements) stays inside the workspace."""
    S, L = splitk_plan(M, N, K)
    assert S > 1
    KS = ceil_div(K, KSTEP)
    tiles_m, tiles_n = ceil_div(M, 256), ceil_div(N, 128)
    T = tiles_m * tiles_n
    c_stride = (M * N + 3) // 4 * 4
    ws_bytes = S * c_stride * 4
    covered = {}
    nwg = min(T * S, 256)
    for wg in range(nwg):
        first, stride, count = ws_tiles(wg, nwg, T * S)
        for i in range(count):
            u = first + i * stride
            tile, sl = u % T, u // T
            k0, k1 = sl * L, min(KS, sl * L + L)
            assert k0 < k1, (u, k0, k1)
            covered.setdefault(tile, []).append((k0, k1))
            tm, tn = grouped_order(tile, tiles_m, tiles_n)
            for w in range(4):
                row0, col0 = tm * 256 + (w >> 1) * 128, tn * 128 + (w & 1) * 64
                if row0 >= M or col0 >= N:
                    continue
                rh, chh = min(M - row0, 128), min(N - col0, 64)
                base = sl * c_stride * 4 + (row0 * N + col0) * 4
                assert base + ((rh - 1) * N + chh) * 4 <= ws_bytes
    assert sorted(covered) == list(range(T))
    for tile, r in covered.items():
        r.sort()
        assert r[0][0] == 0 and r[-1][1] == KS and all(a[1] == b[0] for a, b in zip(r, r[1:])), tile


@pytest.mark.parametrize("G,N,K,offsets", [
    (4, 256, 256, [0, 256, 512, 800, 1024]), (3, 136, 384, [0, 32, 544, 1056]),
    (128, 1536, 2048, None), (128, 2048, 768, None), (3, 256, 256, [-64, 96, 40, 10 ** 6]),
])
def test_grouped_packed_a_segments_read_the_tile_rows(G, N, K, offsets):
    """mxfp8_grouped_gemm_packed: every 8-row segment copy of a group's tile
    reads exactly its rows' 1 KB of packed bytes inside the two-panel
    descriptor (the packed row of global row m0 + 8s), every scale atom its
    rows' 64-byte record, and segments past the group read nothing."""
    import workloads as wl
    if offsets is None:
        rng = np.random.default_rng(G + N)
        route = wl.zipf_topk_routing(rng, 8192, G, 8)
        offsets, _, _ = wl.group_layout(route, G)
    offsets = np.asarray(offsets, np.int64)
    M_total = max(32, int(min(max(offsets.max(), 0), 10 ** 5)) // 32 * 32)
    KS = ceil_div(K, KSTEP)
    for g, m0, m_end in grouped_tiles(offsets, M_total, 256):
        assert m0 % 8 == 0
        (_, base, num, size), (_, sbase, snum, ssize) = packed_a_descriptors(M_total, K, m0)
        assert base + num <= size and sbase + snum <= ssize and num <= 2 ** 31
        for ks in (0, KS - 1):
            segs, atoms = apack_offsets(m0, m_end, K, ks)
            for s_, off in enumerate(segs):
                row = m0 + s_ * 8
                if off is None:
                    assert row >= m_end or s_ * 8 >= 256
                    continue
                assert row < m_end and off + 1024 <= num
                # the packed bytes of global row `row` at k-step ks, as mxfp8_repack lays them out
                assert base + off == (row // 256 * KS + ks) * TILE_BYTES + row % 256 * 128
            for a, off in enumerate(atoms):
                row = m0 + a * 16
                if off is None:
                    assert row >= m_end
                    continue
                assert off + 64 <= snum and sbase + off == (row // 256 * KS + ks) * 1024 + row % 256 // 16 * 64


@pytest.mark.parametrize("batch,rows,cols", [(1, 32, 32), (1, 96, 160), (1, 256, 256), (1, 288, 416),
                                              (1, 512, 384), (1, 8192, 4096), (3, 96, 160), (2, 288, 416)])
def test_quantize_dual_packed_writes_every_byte_once(batch, rows, cols):
    """quantize_dual_packed_kernel's walk over the half panels of both
    layouts of every matrix of the batch: every byte of the axis-1 packed
    layouts (N = rows, K = cols) and of the axis-0 packed layouts (N = cols,
    K = rows) written exactly once, nothing outside them."""
    KS1, KS0 = ceil_div(cols, KSTEP), ceil_div(rows, KSTEP)
    NP1, NP0 = ceil_div(rows, PANEL), ceil_div(cols, PANEL)
    CT = 2 * NP0
    TPM = 2 * NP1 * CT
    ntiles = batch * TPM
    q1 = np.zeros(batch * NP1 * KS1 * TILE_BYTES, np.int32)
    s1 = np.zeros(batch * NP1 * KS1 * 1024, np.int32)
    q0 = np.zeros(batch * NP0 * KS0 * TILE_BYTES, np.int32)
    s0 = np.zeros(batch * NP0 * KS0 * 1024, np.int32)
    t = np.arange(256)
    for idx in range(ntiles):
        b, rr = idx // TPM, idx % TPM
        R0, C0 = rr // CT * 128, rr % CT * 128
        if C0 < KS1 * 128:
            tl = (b * NP1 + R0 // 256) * KS1 + C0 // 128
            half = R0 // 128 % 2
            base = tl * TILE_BYTES + half * 128 * 128
            for u2 in range(2):
                u = u2 * 256 + t
                r, bb = u >> 2, u & 3
                for c in (2 * bb, 2 * bb + 1):
                    off = base + r * 128 + ((c ^ (r & 7)) << 4)
                    for k in range(16):
                        np.add.at(q1, off + k, 1)
                rp = half * 128 + r
                np.add.at(s1, tl * 1024 + (rp >> 4) * 64 + (rp & 15) + 16 * bb, 1)
        if R0 < KS0 * 128:
            tl = (b * NP0 + C0 // 256) * KS0 + R0 // 128
            h = C0 // 128 % 2
            base = tl * TILE_BYTES + h * 128 * 128
            for i in range(4):
                col, j = i * 32 + (t >> 3), t & 7
                off = base + col * 128 + ((j ^ (col & 7)) << 4)
                for k in range(16):
                    np.add.at(q0, off + k, 1)
            for k in range(4):
                np.add.at(s0, (tl * 256 + h * 128 + t[:128]) * 4 + k, 1)
    for a in (q1, s1, q0, s0):
        assert np.all(a == 1), (rows, cols)


@pytest.mark.parametrize("rows,cols", [(32, 32), (96, 160), (256, 256), (288, 416), (67744, 768)])
def test_quantize_dual_grouped_packed_row_grid_written_once(rows, cols):
    """quantize_dual_walk_kernel<.., ROW_PACKED>: the walk over whole panels
    of rows (2 NP(rows) x ceil(cols / 128) tiles) writes every byte of the
    axis-1 packed layout (N = rows, K = cols) exactly once; the tiles past
    the matrix (R0 >= rows) write only that padding."""
    KS1, NP1 = ceil_div(cols, KSTEP), ceil_div(rows, PANEL)
    TC = ceil_div(cols, 128)
    assert TC == KS1
    ntiles = 2 * NP1 * TC
    q1 = np.zeros(NP1 * KS1 * TILE_BYTES // 16, np.int32)
    s1 = np.zeros(NP1 * KS1 * 1024, np.int32)
    t = np.arange(256)
    axis0_tiles = 0
    for idx in range(ntiles):
        R0, C0 = idx // TC * 128, idx % TC * 128
        assert R0 < NP1 * PANEL and C0 < KS1 * 128
        tl = R0 // 256 * KS1 + C0 // 128
        half = R0 // 128 % 2
        base = tl * TILE_BYTES + half * 128 * 128
        for u2 in range(2):
            u = u2 * 256 + t
            r, bb = u >> 2, u & 3
            for c in (2 * bb, 2 * bb + 1):
                off = base + r * 128 + ((c ^ (r & 7)) << 4)
                np.add.at(q1, off // 16, 1)
            rp = half * 128 + r
            np.add.at(s1, tl * 1024 + (rp >> 4) * 64 + (rp & 15) + 16 * bb, 1)
        axis0_tiles += R0 < rows
    assert np.all(q1 == 1) and np.all(s1 == 1), (rows, cols)
    assert axis0_tiles == ceil_div(rows, 128) * TC        # the tiles of the plain walk, once each


def test_quantize_gather_packed_loads_stay_inside():
    """quantize_gather_packed_kernel: every 16-byte load reads a row of x
    named by the index table (inside [0, rows_in)) and columns inside it;
    rows past rows_out and out-of-range indices load nothing."""
    rows_in, cols, rows_out = 37, 288, 300
    rng = np.random.default_rng(5)
    idx = rng.integers(-3, rows_in + 3, rows_out)
    KS = ceil_div(cols, KSTEP)
    lane = np.arange(64)
    bl, half = lane >> 1, lane & 1
    i, kb4 = bl >> 2, bl & 3
    loaded = np.zeros((rows_in, cols), np.int32)
    for st in range(ceil_div(rows_out, PANEL) * 16 * KS):
        atom, ks = st // KS, st % KS
        kcol = ks * 128 + kb4 * 32 + half * 16
        for u in range(4):
            r = atom * 16 + (u >> 1) * 8 + i
            k = kcol + (u & 1) * 8
            src = np.where(r < rows_out, idx[np.minimum(r, rows_out - 1)], -1)
            ok = (src >= 0) & (src < rows_in) & (k < cols)
            assert np.all(k[ok] + 8 <= cols)
            for e in range(8):
                np.add.at(loaded, (src[ok], k[ok] + e), 1)
    # each output row's source elements read exactly once per output row naming it
    want = np.zeros_like(loaded)
    for r in range(rows_out):
        if 0 <= idx[r] < rows_in:
            want[idx[r]] += 1
    assert np.array_equal(loaded, want)


WS_UNITS = 64


@pytest.mark.parametrize("G,N,K,offsets", [
    (4, 256, 256, [0, 256, 512, 800, 1024]), (3, 136, 384, [0, 32, 544, 1056]),
    (5, 200, 128, [0, 0, 96, 96, 384, 640]),             # empty groups, a group ending on a panel edge
    (128, 1536, 2048, None), (128, 2048, 768, None), (3, 256, 256, [-64, 96, 40, 10 ** 6]),
])
def test_ws_grouped_copies_and_stores(G, N, K, offsets):
    """gemm_ws_kernel<.., GROUPED>: with the launcher's bound on the tile
    count, every workgroup's tiles fit its 64-entry table; each tile's A
    segment and scale-atom copies read exactly the packed bytes of its own
    rows (global row m0 + 8s, inside the one- or two-panel descriptor) and
    nothing past its expert; B comes from the expert's panel; and the
    computing waves' stores cover each (row of a group, column) once and no
    row outside the groups."""
    import workloads as wl
    if offsets is None:
        rng = np.random.default_rng(G + N)
        route = wl.zipf_topk_routing(rng, 8192, G, 8)
        offsets, _, _ = wl.group_layout(route, G)
    offsets = np.asarray(offsets, np.int64)
    M_total = max(32, int(min(max(offsets.max(), 0), 10 ** 5)) // 32 * 32)
    # a malformed table (offsets off the 32-row grid or decreasing) only has
    # to keep every descriptor and store inside its buffer
    wellformed = bool(np.all(offsets % 32 == 0) and np.all(np.diff(offsets) >= 0) and offsets[0] >= 0)
    KS, NPa, NP = ceil_div(K, KSTEP), ceil_div(M_total, PANEL), ceil_div(N, PANEL)
    tiles = grouped_tiles(offsets, M_total, 256)
    tiles_m, tiles_n = len(tiles), ceil_div(N, 128)
    T = tiles_m * tiles_n
    bound = (ceil_div(M_total, 256) + G) * tiles_n          # the launcher's tile-count bound
    assert T <= bound
    for cus in (256, 80):
        if bound > (WS_UNITS - 2) * cus:
            continue
        counts = [ws_tiles(wg, cus, T)[2] for wg in range(cus)]
        assert max(counts) <= WS_UNITS, (cus, max(counts))
    lane = np.arange(64)
    row_hits = {}
    for L in range(T):
        tm, tn = grouped_order(L, tiles_m, tiles_n)
        g, m0, m_end = tiles[tm]
        assert 0 <= m0 < m_end <= M_total and (m0 % 32 == 0 or not wellformed)
        pa, a_m0, a_rows = m0 // PANEL, m0 % PANEL, min(m_end - m0, 256)
        na = min(2, NPa - pa)
        abase, anum = pa * KS * TILE_BYTES, na * KS * TILE_BYTES
        sbase, snum = pa * KS * 1024, na * KS * 1024
        assert abase + anum <= NPa * KS * TILE_BYTES and sbase + snum <= NPa * KS * 1024 and anum < 2 ** 31
        for ks in ((0, KS - 1) if wellformed else ()):
            seen = []
            for pw in range(4):
                for i in range(8):
                    seg = i * 4 + pw
                    if seg * 8 >= a_rows:
                        continue                      # kOOB: rows past the expert read zeros
                    r = a_m0 + seg * 8
                    off = (r // PANEL) * KS * TILE_BYTES + ks * TILE_BYTES + (r % PANEL) * 128 + lane * 16
                    assert off.max() + 16 <= anum
                    row = m0 + seg * 8
                    assert row + 8 <= m_end
                    assert abase + off[0] == (row // PANEL * KS + ks) * TILE_BYTES + row % PANEL * 128
                    seen += list(range(row, row + 8))
                ra16 = (pw * 4 + (lane >> 4)) * 16
                ok = ra16 < a_rows
                r = a_m0 + ra16
                soff = (r // PANEL) * KS * 1024 + ks * 1024 + ((r % PANEL) >> 4) * 64 + (lane & 15) * 4
                assert np.all(soff[ok] + 4 <= snum)
                row = m0 + ra16
                assert np.all(row[ok] < m_end)
                assert np.all(sbase + soff[ok] == (row[ok] // PANEL * KS + ks) * 1024 + row[ok] % PANEL // 16 * 64
                              + (lane[ok] & 15) * 4)
            assert sorted(seen) == list(range(m0, m0 + a_rows))
        pb, prow = g * NP + tn * 128 // PANEL, tn * 128 % PANEL
        bbase, bnum = pb * KS * TILE_BYTES + prow * 128, KS * TILE_BYTES - prow * 128
        assert bbase + bnum <= G * NP * KS * TILE_BYTES
        assert (KS - 1) * TILE_BYTES + 15 * 1024 + 1024 <= bnum
        assert pb * KS * 1024 + prow // 16 * 64 + (KS * 1024 - prow // 16 * 64) <= G * NP * KS * 1024
        for w in range(4):
            row0, col0 = m0 + (w >> 1) * 128, tn * 128 + (w & 1) * 64
            if m_end - row0 <= 0 or N - col0 <= 0:
                continue
            rh = min(m_end - row0, 128)
            assert row0 >= 0 and row0 + rh <= M_total
            for rr in range(row0, row0 + rh):
                row_hits[(rr, col0)] = row_hits.get((rr, col0), 0) + 1
    if not wellformed:
        return
    # every row of every group, for every 64-column block, stored exactly once
    want = set()
    for g in range(G):
        lo = min(max(int(offsets[g]), 0), M_total)
        hi = min(max(int(offsets[g + 1]), lo), M_total)
        for rr in range(lo, hi):
            for c0 in range(0, N, 64):
                want.add((rr, c0))
    assert set(row_hits) == want and all(v == 1 for v in row_hits.values())


def _dst_block_of(src, dst, rows, rows_out, r):
    """Mirror of dst_block_of (well-formed tables): destination 32-row block of
    the source block starting at row r, or -1."""
    if r >= rows:
        return -1
    G = len(src) - 1
    for g in range(G):
        lo, hi = min(max(src[g], 0), rows), min(max(src[g + 1], 0), rows)
        if lo <= r < hi:
            dlo = min(max(dst[g], 0), rows_out)
            dhi = min(max(dst[g + 1], dlo), rows_out)
            if lo % 32 or dlo % 32:
                return -1
            d = dlo + (r - lo)
            return d // 32 if d + 32 <= dhi else -1
    return -1


@pytest.mark.parametrize("tokens,experts,topk,cols,row_grid", [(64, 8, 2, 64, True), (512, 16, 4, 288, False),
                                                               (8192, 128, 8, 768, True)])
def test_quantize_dual_grouped_packed_col_grid_written_once(tokens, experts, topk, cols, row_grid):
    """mxfp8_quantize_dual_grouped_packed's regrouped grid in the packed layout
    (N = cols, K = rows_out): the walk's stores (destination block d of column
    f at k-step d / 4, K-block d % 4, chunks 2 (d % 4) + h at slot c ^ (f % 8))
    and zero_dst_pads_packed_kernel's (pad blocks in every column, the layout's
    padding rows and blocks) write every byte exactly once, and the pad kernel's
    scale codes are 0 for pad blocks, 127 for padding."""
    import workloads as wl
    rng = np.random.default_rng(tokens + cols)
    route = wl.zipf_topk_routing(rng, tokens, experts, topk)
    src, _, _ = wl.group_layout(route, experts)
    src = [int(v) for v in src]
    sizes = np.diff(src)
    dst = [0] + list(np.cumsum(-(-sizes // 128) * 128))
    dst = [int(v) for v in dst]
    rows, rows_out = src[-1], dst[-1] + 64               # trailing blocks in no group
    KS, NP = ceil_div(rows_out, 128), ceil_div(cols, PANEL)
    q = np.zeros(NP * KS * TILE_BYTES // 16, np.int32)
    s = np.zeros(NP * KS * 1024, np.int32)
    scode = np.full(NP * KS * 1024, -1, np.int64)
    f_all = np.arange(NP * PANEL)

    def mark(f, d, code=None):
        tl = (f // PANEL) * KS + d // 4
        frow = f % PANEL
        for h in range(2):
            c = 2 * (d % 4) + h
            np.add.at(q, (tl * TILE_BYTES + frow * 128 + ((c ^ (frow & 7)) << 4)) // 16, 1)
        si = tl * 1024 + (frow >> 4) * 64 + (frow & 15) + 16 * (d % 4)
        np.add.at(s, si, 1)
        if code is not None:
            scode[si] = code
    # the walk: source row blocks of the tiles with R0 < rows (both walk shapes cover the same ones)
    for r in range(0, ceil_div(rows, 128) * 128, 32):
        d = _dst_block_of(src, dst, rows, rows_out, r)
        if d >= 0:
            mark(f_all[:cols], d)
    # the pad kernel
    for d in range(KS * 4):
        d0 = d * 32
        if d0 >= rows_out:
            kind = 2
        else:
            found = None
            for g in range(experts):
                dlo = min(max(dst[g], 0), rows_out)
                dhi = min(max(dst[g + 1], dlo), rows_out)
                if dlo <= d0 < dhi:
                    found = (dlo, dhi, src[g + 1] - src[g])
                    break
            kind = 0 if found and d0 - found[0] < found[2] and d0 + 32 <= found[1] else 1
        fs = f_all if kind else f_all[cols:]
        if fs.size:
            mark(fs, d, np.where((kind == 1) & (fs < cols), 0, 127))
    assert np.all(q == 1) and np.all(s == 1), (tokens, cols)
    assert set(np.unique(scode)) <= {-1, 0, 127}


@pytest.mark.parametrize("G,M,N,sizes", [(4, 256, 320, [128, 0, 384, 256]), (3, 300, 132, [0, 0, 128]),
                                         (128, 1536, 2048, None), (128, 2048, 768, None)])
def test_ws_grouped_k_units(G, M, N, sizes):
    """gemm_ws_kernel<.., GK>: units = (expert, 256x128 tile) dealt in dispatch
    order (workgroup j: units j, j + grid, ...), each over its expert's k-steps [o_g / 128, ceil(o_{g+1} / 128)) of the
    packed token axis (an expert without tokens: one step, every copy out of
    range); the A / B panels' copies stay inside the packed operands and each
    element of C[g] is stored exactly once, at g * M * N."""
    import workloads as wl
    if sizes is None:
        rng = np.random.default_rng(G + N)
        route = wl.zipf_topk_routing(rng, 8192, G, 8)
        off32, _, _ = wl.group_layout(route, G)
        sz = np.diff(off32)
        sizes = list(-(-sz // 128) * 128)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    T = max(int(offs[-1]), 128)
    KS, NPm, NPn = ceil_div(T, KSTEP), ceil_div(M, PANEL), ceil_div(N, PANEL)
    tiles_m, tiles_n = ceil_div(M, 256), ceil_div(N, 128)
    Tt = tiles_m * tiles_n
    units = G * Tt
    nwg = min(units, 256)
    seen = []
    steps = 0
    hits = np.zeros(G * M * N if G * M * N <= 1 << 27 else 1, np.int32)
    for wg in range(nwg):
        first, stride = wg, nwg                   # dispatch order
        count = -(-(units - first) // stride) if first < units else 0
        for i in range(count):
            u = first + i * stride
            seen.append(u)
            g, tile = u // Tt, u % Tt
            lo, hi = min(max(offs[g], 0), T), min(max(offs[g + 1], offs[g]), T)
            k0, k1 = lo // 128, -(-hi // 128)
            empty = k1 == k0
            if empty:
                k1 = k0 + 1
            assert 0 <= k0 < k1 <= max(KS, 1) or (empty and k0 <= KS)
            steps += k1 - k0
            tm, tn = grouped_order(tile, tiles_m, tiles_n)
            pb, prow = tn * 128 // PANEL, tn * 128 % PANEL
            # descriptors: A panel tm, B half panel, each over all KS k-steps
            assert (tm + 1) * KS * TILE_BYTES <= NPm * KS * TILE_BYTES
            assert pb * KS * TILE_BYTES + prow * 128 + (KS * TILE_BYTES - prow * 128) <= NPn * KS * TILE_BYTES
            if not empty:
                # the last copy of the unit's last step inside its descriptor
                assert (k1 - 1) * TILE_BYTES + 31 * 1024 + 1024 <= KS * TILE_BYTES
                assert (k1 - 1) * TILE_BYTES + 15 * 1024 + 1024 <= KS * TILE_BYTES - prow * 128
            if hits.size > 1:
                for w in range(4):
                    row0, col0 = tm * 256 + (w >> 1) * 128, tn * 128 + (w & 1) * 64
                    if row0 >= M or col0 >= N:
                        continue
                    rh, ch = min(M - row0, 128), min(N - col0, 64)
                    base = g * M * N + row0 * N + col0
                    for r in range(rh):
                        hits[base + r * N: base + r * N + ch] += 1
    assert sorted(seen) == list(range(units))
    if hits.size > 1:
        assert np.all(hits == 1)
