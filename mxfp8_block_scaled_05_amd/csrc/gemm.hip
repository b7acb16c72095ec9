// Block-scaled MXFP8 GEMM on gfx950 scaled MFMA:  C[M][N] = A[M][K] * B[N][K]^T.
//
// The page describes MXFP8 as the block-scaled FP8 whose per-block scales the
// matrix instruction takes as operands ("End-to-End MXFP8 RL on Blackwell"
// (verl blog), section "The pipeline", paragraph "The format").  On CDNA4 the
// matching instruction is V_MFMA_SCALE_F32_16X16X128_F8F6F4: a 16x16 output
// tile, K = 128 per instruction (four 32-element MX blocks), each lane
// supplying 32 K values of one row plus one E8M0 scale byte; the scale of
// lane group s (= lane / 16) applies to block s.  So the scales never leave
// their byte form and no rescaling arithmetic runs outside the matrix core.
//
// Structure (one workgroup = 8 waves = one BM x BN output tile):
//  - K advances in steps of 128.  The A and B tiles of a step and their
//    scale bytes are staged in LDS with buffer_load ... lds (global -> LDS,
//    no VGPR round trip) issued as inline asm, in an NST-stage ring: the
//    copies for step k+NST-1 stream in while step k feeds the MFMAs.  Every
//    wave issues the same number of copies per step, so one immediate
//    s_waitcnt vmcnt(n) + barrier per step waits for exactly the step needed.
//  - LDS rows are 128 B (one step); the 16-byte chunk c of row r sits at slot
//    c ^ f(r % 16), which makes the ds_read_b128 of 16 rows at one chunk bank
//    conflict free.  Canonical operands are swizzled by choosing each lane's
//    source address; packed weights (mxfp8_repack) are already stored in this
//    image, so their copy is linear.
//  - Out-of-range rows and the K tail read as zeros through the buffer
//    resource's range check (never a memory access out of bounds).
//  - 8 waves (two per SIMD) form a 2x4 grid; each wave owns (BM/2) x (BN/4)
//    of C as 16x16 MFMA tiles accumulated in fp32.
//  - Tiles are mapped XCD-aware: the hardware deals workgroups round-robin to
//    the 8 XCDs, so workgroup ids are renumbered to give each XCD a
//    contiguous range of tiles, ordered in groups of GROUP_M tile-rows so
//    tiles resident on one XCD share A rows and B columns in its L2.
//  - Grouped (MoE) mode reads the per-expert row offsets on the device and
//    locates each tile's expert with a wave-wide prefix scan.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

struct GemmParams {
    const uint8_t *a_q;
    const uint8_t *a_s;
    const uint8_t *b_q;
    const uint8_t *b_s;
    void *c;
    int64_t M, N, K;        // dense: M rows; grouped: M = M_total
    int tiles_m, tiles_n;   // grid tile counts (grouped: upper bound for m)
    const int32_t *offsets;  // grouped only
    int G;
    int KS, NP;              // k-steps, packed panels of B
};

constexpr int kGroupM = 8;
// s_waitcnt immediate for gfx9 with expcnt and lgkmcnt left at their maximum:
// vmcnt(n) for n < 64 (bits [3:0] and [15:14])
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Buffer descriptor in SGPRs for inline asm: base, stride 0, num_records =
// bytes (range-checked: out-of-range lanes read zeros), 32-bit data format.
__device__ __forceinline__ v4i make_srd(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    v4i r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = 0x00020000;
    return r;
}

// LDS byte address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p;
}

// 4 bytes per lane, global -> LDS at m0 + 4 * lane (one wave = 256 B).
__device__ __forceinline__ void dma4(v4i srd, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(srd), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

// 16 bytes per lane, global -> LDS at m0 + 16 * lane (one wave = 1 KB).
__device__ __forceinline__ void dma16(v4i srd, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(srd), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}
// 8 waves (two per SIMD) in a 2 (M) x 4 (N) grid: while one wave of a SIMD
// waits on LDS fragment reads or the barrier, the other keeps its MFMAs issuing.
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;

// Operand fragment of one 16-row x 128-K MFMA tile.  The scaled MFMA reads
// lane group j = lane/16 as two 16-byte K slices, K = 16j..16j+15 (bytes 0-15)
// and K = 64+16j..64+16j+15 (bytes 16-31), while the scale byte of lane group
// s covers the 32-element block K = 32s..32s+31; so lane groups 2t and 2t+1
// together carry block t (first half) and block t+2 (second half), and the
// scale of block s is simply supplied by lane group s.
__device__ __forceinline__ v8i lds_frag(const uint8_t *base, int lane) {
    const int row = lane & 15, jj = lane >> 4;
    const uint32_t f = swz((uint32_t)row);
    const uint8_t *r = base + row * 128;
    const v4i lo = *reinterpret_cast<const v4i *>(r + ((jj ^ f) * 16));
    const v4i hi = *reinterpret_cast<const v4i *>(r + (((4 + jj) ^ f) * 16));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// renumber so that each XCD (workgroup id mod 8) receives a contiguous range
__device__ __forceinline__ int xcd_logical(int wg, int nwg) {
    const int q = nwg / 8, r = nwg % 8, x = wg % 8;
    return x * q + (x < r ? x : r) + wg / 8;
}

__device__ __forceinline__ void grouped_order(int logical, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int per_group = kGroupM * tiles_n;
    const int gid = logical / per_group;
    const int first = gid * kGroupM;
    const int gsz = min(tiles_m - first, kGroupM);
    const int in = logical % per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

// Find the expert owning global m-tile `tm` (tiles of BM rows, counted over the
// groups in order).  Offsets are clamped into [0, M_total] and made
// non-decreasing, so a malformed table can only drop work, never address
// outside the operands.  Returns -1 if `tm` is past the last tile.
template <int BM>
__device__ int find_group(const int32_t *off, int G, int64_t M_total, int tm, int lane, int64_t &lo,
                          int64_t &hi, int &tile_in_group) {
    int base = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        int64_t lo_g = 0, hi_g = 0;
        int t = 0;
        if (g < G) {
            lo_g = off[g];
            hi_g = off[g + 1];
            lo_g = lo_g < 0 ? 0 : (lo_g > M_total ? M_total : lo_g);
            hi_g = hi_g < lo_g ? lo_g : (hi_g > M_total ? M_total : hi_g);
            t = (int)((hi_g - lo_g + BM - 1) / BM);
        }
        int incl = t;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        const int excl = incl - t;
        const bool hit = g < G && tm >= base + excl && tm < base + incl;
        const unsigned long long mask = __ballot(hit);
        if (mask) {
            const int src = __ffsll((long long)mask) - 1;
            lo = __shfl(lo_g, src);
            hi = __shfl(hi_g, src);
            tile_in_group = tm - base - __shfl(excl, src);
            return g0 + src;
        }
        base += __shfl(incl, 63);
    }
    return -1;
}

template <int BM, int BN, bool BPACK, bool OUT_BF16, bool GROUPED, bool KALIGN, int NST>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
    constexpr int WTM = BM / kWavesM, WTN = BN / kWavesN;   // wave tile
    constexpr int FM = WTM / 16, FN = WTN / 16;            // MFMA tiles per wave (rows, cols)
    // LDS: NST stages of [A tile | B tile | A scales | B scales].  A scales
    // (K % 128 == 0) are a dword per row per step; B scales are the packed
    // layout's 64 bytes per 16-row atom per step, or (canonical B, K % 128
    // == 0) a dword per row.  With K % 128 != 0, A (and canonical B) scale
    // bytes come through registers instead (compiler-visible byte loads).
    constexpr bool SA_LDS = KALIGN;
    constexpr bool SB_LDS = BPACK || KALIGN;
    constexpr int TILE = (BM + BN) * 128;
    constexpr int SA_OFF = TILE;
    constexpr int SB_OFF = SA_OFF + (SA_LDS ? BM * 4 : 0);
    constexpr int STAGE = SB_OFF + (SB_LDS ? BN * 4 : 0);
    static_assert(NST * STAGE <= 160 * 1024, "LDS budget");
    static_assert(KALIGN || NST == 2, "register-fed scales are fetched one step ahead");
    // copies per wave per step: tile segments plus one A- and one B-scale copy
    constexpr int CPW = BM / (8 * kWaves) + BN / (8 * kWaves) + (SA_LDS ? 1 : 0) + (SB_LDS ? 1 : 0);
    static_assert(CPW * (NST - 2) < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * STAGE];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wm = w / kWavesN, wn = w % kWavesN;

    int tm, tn;
    grouped_order(xcd_logical(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
    if (tm >= p.tiles_m || tn >= p.tiles_n) return;

    const int64_t K = p.K, N = p.N;
    const int64_t KB = K / 32;        // scale bytes per row
    int64_t m0, m_end;
    int64_t g = 0;
    if constexpr (GROUPED) {
        int64_t lo, hi;
        int tig;
        const int gg = find_group<BM>(p.offsets, p.G, p.M, tm, lane, lo, hi, tig);
        if (gg < 0) return;
        g = gg;
        m0 = lo + (int64_t)tig * BM;
        m_end = hi;
    } else {
        m0 = (int64_t)tm * BM;
        m_end = p.M;
    }
    const int64_t n0 = (int64_t)tn * BN;
    const int rows_a = (int)min((int64_t)BM, m_end - m0);

    // ---- operand descriptors (SGPRs, for the inline-asm copies): each one
    //      spans exactly the bytes of this tile, so out-of-range lanes read 0
    const v4i ra = make_srd(p.a_q + m0 * K, (uint32_t)(rows_a * K));
    const v4i rsa = make_srd(p.a_s + m0 * KB, (uint32_t)(rows_a * KB));
    v4i rb, rsb;
    if constexpr (BPACK) {
        const int64_t panel = n0 / kPanelRows, prow = n0 % kPanelRows;
        const uint8_t *bt = p.b_q + ((g * p.NP + panel) * p.KS) * kTileBytes + prow * 128;
        rb = make_srd(bt, (uint32_t)((int64_t)p.KS * kTileBytes - prow * 128));
        const uint8_t *bs = p.b_s + ((g * p.NP + panel) * p.KS) * kScaleStepBytes + (prow / 16) * 64;
        rsb = make_srd(bs, (uint32_t)((int64_t)p.KS * kScaleStepBytes - (prow / 16) * 64));
    } else {
        const int rows_b = (int)min((int64_t)BN, N - n0);
        rb = make_srd(p.b_q + n0 * K, (uint32_t)(rows_b * K));
        rsb = make_srd(p.b_s + n0 * KB, (uint32_t)(rows_b * KB));
    }
    // the same ranges as compiler-visible resources, for the byte-granular
    // scale loads of the K % 128 != 0 path
    const __amdgpu_buffer_rsrc_t rsa_c = make_rsrc(p.a_s + m0 * KB, (uint32_t)(rows_a * KB));
    const __amdgpu_buffer_rsrc_t rsb_c =
        make_rsrc(p.b_s + (BPACK ? 0 : n0 * KB), BPACK ? 0u : (uint32_t)(min((int64_t)BN, N - n0) * KB));
    const int Ki = (int)K, KBi = (int)KB;
    const uint32_t lds0 = lds_addr(smem);

    // ---- global -> LDS copies of k-step ks into stage st: CPW per wave
    auto issue = [&](int ks, int st) {
        const uint32_t sbase = lds0 + st * STAGE;
#pragma unroll
        for (int i = 0; i < BM / (8 * kWaves); ++i) {
            const int seg = i * kWaves + w;            // 1 KB LDS segment = 8 rows
            const int rr = seg * 8 + (lane >> 3);
            const int c = (lane & 7) ^ (int)swz((uint32_t)rr);
            const int kk = ks * 128 + c * 16;
            const uint32_t off = kk < Ki ? (uint32_t)(rr * Ki + kk) : kOOB;
            dma16(ra, off, sbase + seg * 1024);
        }
#pragma unroll
        for (int i = 0; i < BN / (8 * kWaves); ++i) {
            const int seg = i * kWaves + w;
            uint32_t off;
            if constexpr (BPACK) {
                off = (uint32_t)ks * (uint32_t)kTileBytes + seg * 1024 + lane * 16;
            } else {
                const int rr = seg * 8 + (lane >> 3);
                const int c = (lane & 7) ^ (int)swz((uint32_t)rr);
                const int kk = ks * 128 + c * 16;
                off = kk < Ki ? (uint32_t)(rr * Ki + kk) : kOOB;
            }
            dma16(rb, off, sbase + BM * 128 + seg * 1024);
        }
        // scale copies: 256 B segments.  With more than two stages every wave
        // issues one of each (a wave beyond the segment count repeats one:
        // identical bytes to the same place) so the per-wave count CPW, and
        // with it the loop's vmcnt immediate, is uniform; with two stages
        // (vmcnt(0)) only the waves with a segment of their own copy.
        if constexpr (SA_LDS) {
            if (NST > 2 || w < BM / 64) {
                const int seg = w % (BM / 64);
                const int rr = seg * 64 + lane;
                dma4(rsa, (uint32_t)(rr * KBi + ks * 4), sbase + SA_OFF + seg * 256);
            }
        }
        if constexpr (SB_LDS) {
            if (NST > 2 || w < BN / 64) {
                const int seg = w % (BN / 64);
                uint32_t off;
                if constexpr (BPACK) off = (uint32_t)(ks * kScaleStepBytes + seg * 256 + lane * 4);
                else off = (uint32_t)((seg * 64 + lane) * KBi + ks * 4);
                dma4(rsb, off, sbase + SB_OFF + seg * 256);
            }
        }
    };

    // ---- K % 128 != 0: A (and canonical B) scale bytes by compiler-visible
    //      loads, one step ahead (the K tail's blocks read as 0)
    const int lrow = lane & 15, lblk = lane >> 4;
    auto fetch_sa = [&](int ks, uint32_t *dst) {
        const int blk = ks * 4 + lblk;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int rr = wm * WTM + i * 16 + lrow;
            const uint32_t off = blk < KBi ? (uint32_t)(rr * KBi + blk) : kOOB;
            dst[i] = __builtin_amdgcn_raw_buffer_load_b8(rsa_c, off, 0, 0);
        }
    };
    auto fetch_sb = [&](int ks, uint32_t *dst) {
        const int blk = ks * 4 + lblk;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int rr = wn * WTN + j * 16 + lrow;
            const uint32_t off = blk < KBi ? (uint32_t)(rr * KBi + blk) : kOOB;
            dst[j] = __builtin_amdgcn_raw_buffer_load_b8(rsb_c, off, 0, 0);
        }
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint32_t sa_cur[FM], sa_nxt[FM], sb_cur[FN], sb_nxt[FN];
    const int KS = p.KS;
    if constexpr (!SA_LDS) fetch_sa(0, sa_nxt);
    if constexpr (!SB_LDS) fetch_sb(0, sb_nxt);
#pragma unroll
    for (int s0 = 0; s0 < NST - 1; ++s0)
        if (s0 < KS) issue(s0, s0);

    for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks % NST;
        // this step's copies have landed (this wave's: vmcnt, letting the
        // copies of later steps stay in flight; everyone's: the barrier), and
        // every wave is done reading the stage the next issue overwrites
        if constexpr (NST >= 3) {
            if (ks + NST - 2 < KS) __builtin_amdgcn_s_waitcnt(waitcnt_vm(CPW * (NST - 2)));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        __syncthreads();
        if constexpr (!SA_LDS || !SB_LDS) {
            if constexpr (!SA_LDS) {
#pragma unroll
                for (int i = 0; i < FM; ++i) sa_cur[i] = sa_nxt[i];
            }
            if constexpr (!SB_LDS) {
#pragma unroll
                for (int j = 0; j < FN; ++j) sb_cur[j] = sb_nxt[j];
            }
            if (ks + 1 < KS) {
                if constexpr (!SA_LDS) fetch_sa(ks + 1, sa_nxt);
                if constexpr (!SB_LDS) fetch_sb(ks + 1, sb_nxt);
            }
        }
        if (ks + NST - 1 < KS) issue(ks + NST - 1, (ks + NST - 1) % NST);

        const uint8_t *st = smem + cur * STAGE;
        const uint8_t *sa = st + wm * WTM * 128;
        const uint8_t *sb = st + BM * 128 + wn * WTN * 128;
        int sas[FM], sbs[FN];
        // the MFMA reads bits [7:0] of each scale register (op_sel 0)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if constexpr (SA_LDS) sas[i] = st[SA_OFF + (wm * WTM + i * 16 + lrow) * 4 + lblk];
            else sas[i] = (int)(sa_cur[i] & 0xFFu);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (BPACK) sbs[j] = st[SB_OFF + (wn * FN + j) * 64 + lane];
            else if constexpr (SB_LDS) sbs[j] = st[SB_OFF + (wn * WTN + j * 16 + lrow) * 4 + lblk];
            else sbs[j] = (int)(sb_cur[j] & 0xFFu);
        }
        v8i bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = lds_frag(sb + j * 16 * 128, lane);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const v8i af = lds_frag(sa + i * 16 * 128, lane);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af, bf[j], acc[i][j], 0, 0, 0, sas[i], 0, sbs[j]);
        }
    }

    // ---- epilogue: lane holds C[4*(lane/16) + r][lane % 16] of each 16x16 tile
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = n0 + wn * WTN + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * WTM + i * 16 + (lane >> 4) * 4 + r;
                if (row < m_end && col < N) {
                    if constexpr (OUT_BF16)
                        static_cast<uint16_t *>(p.c)[row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
                    else
                        static_cast<float *>(p.c)[row * N + col] = acc[i][j][r];
                }
            }
        }
    }
}

// Pipeline depth.  Two stages measured fastest on MI355X for every tile shape
// here (a third stage keeps more copies in flight but did not shorten the
// qkv GEMM); the NST > 2 path is kept for tuning.
template <int BM, int BN>
constexpr int stages_for() { return 2; }

template <int BM, int BN, bool GROUPED, bool KALIGN, int NST>
static hipError_t launch_cfg2(const GemmParams &p, bool b_packed, bool c_bf16, int nwg, hipStream_t s) {
    dim3 grid((unsigned)nwg), block(kThreads);
    if (b_packed) {
        if (c_bf16) hipLaunchKernelGGL((gemm_kernel<BM, BN, true, true, GROUPED, KALIGN, NST>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((gemm_kernel<BM, BN, true, false, GROUPED, KALIGN, NST>), grid, block, 0, s, p);
    } else {
        if (c_bf16) hipLaunchKernelGGL((gemm_kernel<BM, BN, false, true, GROUPED, KALIGN, NST>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((gemm_kernel<BM, BN, false, false, GROUPED, KALIGN, NST>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

template <int BM, int BN, bool GROUPED>
static hipError_t launch_cfg(const GemmParams &p, bool b_packed, bool c_bf16, int nwg, hipStream_t s) {
    if (p.K % 128 == 0) return launch_cfg2<BM, BN, GROUPED, true, stages_for<BM, BN>()>(p, b_packed, c_bf16, nwg, s);
    return launch_cfg2<BM, BN, GROUPED, false, 2>(p, b_packed, c_bf16, nwg, s);
}

hipError_t launch_gemm(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                       const uint8_t *b_s, bool b_packed, int64_t M, int64_t N, int64_t K, void *c,
                       bool c_bf16, hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = c;
    p.M = M; p.N = N; p.K = K;
    p.KS = (int)packed_ksteps(K);
    p.NP = (int)packed_panels(N);
    p.G = 1;
    p.offsets = nullptr;
    const int cus = device_cu_count();
    // 256x256 tiles unless that leaves the last wave of tiles badly filled,
    // then 256x128 (twice the tiles, and a three-stage pipeline).
    const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t waves256 = ceil_div(t256, cus);
    const double fill256 = (double)t256 / (double)(waves256 * cus);
    if (fill256 >= 0.85 || N <= 128) {
        p.tiles_m = (int)ceil_div(M, 256);
        p.tiles_n = (int)ceil_div(N, 256);
        return launch_cfg<256, 256, false>(p, b_packed, c_bf16, p.tiles_m * p.tiles_n, stream);
    }
    p.tiles_m = (int)ceil_div(M, 256);
    p.tiles_n = (int)ceil_div(N, 128);
    return launch_cfg<256, 128, false>(p, b_packed, c_bf16, p.tiles_m * p.tiles_n, stream);
}

hipError_t launch_grouped_gemm(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                               const uint8_t *b_s, const int32_t *offsets, int64_t G,
                               int64_t M_total, int64_t N, int64_t K, void *c, bool c_bf16,
                               hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = c;
    p.M = M_total; p.N = N; p.K = K;
    p.KS = (int)packed_ksteps(K);
    p.NP = (int)packed_panels(N);
    p.G = (int)G;
    p.offsets = offsets;
    constexpr int BM = 128, BN = 256;
    p.tiles_m = (int)(ceil_div(M_total, BM) + G);
    p.tiles_n = (int)ceil_div(N, BN);
    return launch_cfg<BM, BN, true>(p, true, c_bf16, p.tiles_m * p.tiles_n, stream);
}

}  // namespace mx
