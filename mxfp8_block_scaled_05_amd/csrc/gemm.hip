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
//    no VGPR round trip) issued as inline asm and awaited explicitly
//    (s_waitcnt vmcnt + barrier), so the compiler never orders its own waits
//    behind them.
//  - A 2-stage ring with one barrier at the top of each step.
//  - LDS rows are 128 B (one step); the 16-byte chunk c of row r sits at slot
//    c ^ (r % 8), which makes the ds_read_b128 of 16 rows at one chunk bank
//    conflict free (swz).  Canonical operands are swizzled by choosing each lane's
//    source address; packed weights (mxfp8_repack) are already stored in this
//    image, so their copy is linear.
//  - Out-of-range rows and the K tail read as zeros through the buffer
//    resource's range check (never a memory access out of bounds).
//  - 8 waves (two per SIMD) form a WM x (8/WM) grid; each wave owns a
//    (BM/WM) x (BN/(8/WM)) block of C as 16x16 MFMA tiles accumulated in fp32.
//  - Tiles are mapped XCD-aware: the hardware deals workgroups round-robin to
//    the 8 XCDs, so workgroup ids are renumbered to give each XCD a
//    contiguous range of tiles, ordered in groups of GROUP_M tile-rows so
//    tiles resident on one XCD share A rows and B columns in its L2.
//  - Grouped (MoE) mode reads the per-expert row offsets on the device and
//    locates each tile's expert with a wave-wide prefix scan.
#include "mx_device.hpp"
#include "mx_launch.hpp"

#include <algorithm>
#include <mutex>

namespace mx {

// Device scratch of the allocation-free split-K call: the fp32 partial tiles
// of every K slice.  A split plan keeps slices x tiles within one round of
// the CUs and each tile covers at most 256 x 128 outputs, so on a 256-CU
// device a plan needs at most 256 x 32768 x 4 bytes plus the per-slice
// rounding to 16 bytes.  Each device the library runs on holds its own copy
// of this array until the process ends.
constexpr size_t kSplitScratchBytes = ((size_t)32 << 20) + 4096;
static __device__ __align__(256) uint8_t scratch[kSplitScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void *g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
}  // namespace

// The device address of `scratch` on the current device.  In host code the
// array's name is only a host-side stand-in, so its address is looked up once
// per device (with that device current) and the looked-up pointer is what
// kernels receive.
hipError_t splitk_scratch(void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev]() {
        void *p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_err[dev] = r;
        g_scratch_ptr[dev] = r == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *ptr = g_scratch_ptr[dev];
    *bytes = kSplitScratchBytes;
    return hipSuccess;
}

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
    // canonical operand row strides in bytes (elements, scales): K and K/32,
    // except in grouped-K mode where rows span all groups' tokens
    int64_t lda, lsa, ldb, lsb;
    int64_t c_stride;        // grouped-K: elements of one group's C
    int mix_big, mix_big_cols;   // mixed dense launch: 256x256 tiles and their tile columns
    int splits, split_steps;     // split-K: K slices and k-steps per slice
};

constexpr int kGroupM = 4;
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
// 8 waves (two per SIMD): while one wave of a SIMD waits on LDS fragment
// reads or a barrier, the other keeps its MFMAs issuing.
constexpr int kWaves = 8;
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

// Total m-tiles of BM rows over all groups (clamped like find_group), the same
// in every lane.
template <int BM>
__device__ int count_group_tiles(const int32_t *off, int G, int64_t M_total, int lane) {
    int total = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        int t = 0;
        if (g < G) {
            int64_t lo = off[g], hi = off[g + 1];
            lo = lo < 0 ? 0 : (lo > M_total ? M_total : lo);
            hi = hi < lo ? lo : (hi > M_total ? M_total : hi);
            t = (int)((hi - lo + BM - 1) / BM);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d);
        total += t;
    }
    return total;
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

// Per-tile state and the operations of one k-step, shared by both pipelines.
template <int BM, int BN, int WM, bool BPACK, bool KALIGN, bool SAC = false, bool APACK = false>
struct TileOps {
    static constexpr int WN = kWaves / WM;
    static constexpr int WTM = BM / WM, WTN = BN / WN;       // wave tile
    static constexpr int FM = WTM / 16, FN = WTN / 16;      // MFMA tiles per wave
    // LDS stage: [A tile | B tile | A scales | B scales].  A scales (K % 128
    // == 0) are a dword per row per step; B scales are the packed layout's
    // 64 bytes per 16-row atom per step, or (canonical B, K % 128 == 0) a
    // dword per row.  With K % 128 != 0, A (and canonical B) scale bytes come
    // through registers instead (compiler-visible byte loads).  SAC: the A
    // scales come instead from a chunk buffer outside the stage ring that
    // holds 8 k-steps of them (32 bytes per row), copied once per 8 steps.
    static_assert(!SAC || KALIGN, "chunked A scales need K % 128 == 0");
    // APACK: A in the packed layout too (panels of 256 rows, each k-step's
    // 32 KB tile contiguous, rows' 16-byte chunks already in their LDS slots;
    // the step's scales a 1 KB per-lane tile), copied exactly as packed B
    static_assert(!APACK || (BPACK && KALIGN && !SAC && BM == 256), "packed A: packed B, K % 128 == 0, 256-row tiles");
    static constexpr bool SA_LDS = KALIGN && !SAC;
    static constexpr bool SA_REG = !KALIGN;
    static constexpr int kChunkSteps = 8;
    static constexpr int CHUNK = BM * 4 * kChunkSteps;     // bytes of one chunk buffer
    // SBC: canonical B scales of 256-row B tiles chunked the same way
    static constexpr bool SBC = SAC && !BPACK && BN == 256;
    static constexpr bool SB_LDS = BPACK || (KALIGN && !SBC);
    static constexpr bool SB_REG = !BPACK && !KALIGN;
    static constexpr int CHUNK_B = SBC ? BN * 4 * kChunkSteps : 0;
    static constexpr int TILE = (BM + BN) * 128;
    static constexpr int SA_OFF = TILE;
    static constexpr int SB_OFF = SA_OFF + (SA_LDS ? BM * 4 : 0);
    static constexpr int STAGE = SB_OFF + (SB_LDS ? BN * 4 : 0);
    static_assert(FM >= 2 && FN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "copy segments");

    v4i ra, rsa, rb, rsb;
    __amdgpu_buffer_rsrc_t rsa_c, rsb_c;
    int Ki, KBi, lane, w, wm, wn, lrow, lblk;
    int rows_a, rows_b;        // rows of the A and B tiles inside the operands
    int a_r0, KSa;             // APACK: the tile's first row in its first panel; k-steps per panel
    int lda, lsa, ldb, lsb;    // row strides of canonical operands (bytes)
    uint32_t lds0;

    // kbase / kbound: this tile's K range [kbase, kbase + kbound) of each
    // canonical row (all of K unless in grouped-K mode)
    __device__ __forceinline__ void init(const GemmParams &p, int64_t m0, int64_t m_end, int64_t n0, int64_t g,
                         const uint8_t *smem, int64_t kbase = 0, int64_t kbound = -1) {
        const int64_t K = kbound < 0 ? p.K : kbound, N = p.N, KB = K / 32;
        lane = threadIdx.x & 63;
        w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        wm = w / WN;
        wn = w % WN;
        lrow = lane & 15;
        lblk = lane >> 4;
        Ki = (int)K;
        KBi = (int)KB;
        lda = (int)p.lda;
        lsa = (int)p.lsa;
        ldb = (int)p.ldb;
        lsb = (int)p.lsb;
        lds0 = lds_addr(smem);
        const int64_t rows_a = min((int64_t)BM, m_end - m0);
        this->rows_a = (int)rows_a;
        this->rows_b = (int)min((int64_t)BN, N - n0);
        // each descriptor spans exactly this tile's bytes (from its first row's
        // K range start to its last row's K range end): out-of-range lanes read 0
        const uint32_t a_bytes = (uint32_t)((rows_a - 1) * p.lda + K);
        const uint32_t as_bytes = (uint32_t)((rows_a - 1) * p.lsa + KB);
        if constexpr (APACK) {
            // A's panels from m0 / 256 on (K from 0: kbase == 0 for packed A).
            // Dense tiles start a panel; grouped tiles start at any row of a
            // group (a multiple of 32) and may run into the next panel, so the
            // descriptors span two panels where there are two, and each
            // 8-row copy segment / 16-row scale atom finds its own panel row.
            const int64_t pa = m0 / kPanelRows, np = min((int64_t)2, (p.M + kPanelRows - 1) / kPanelRows - pa);
            a_r0 = (int)(m0 % kPanelRows);
            KSa = p.KS;
            ra = make_srd(p.a_q + pa * p.KS * kTileBytes, (uint32_t)(np * p.KS * kTileBytes));
            rsa = make_srd(p.a_s + pa * p.KS * kScaleStepBytes, (uint32_t)(np * p.KS * kScaleStepBytes));
            rsa_c = make_rsrc(p.a_s, 0u);
            (void)a_bytes;
            (void)as_bytes;
        } else {
            ra = make_srd(p.a_q + m0 * p.lda + kbase, a_bytes);
            rsa = make_srd(p.a_s + m0 * p.lsa + kbase / 32, as_bytes);
            rsa_c = make_rsrc(p.a_s + m0 * p.lsa + kbase / 32, as_bytes);
        }
        if constexpr (BPACK) {
            // packed B from k-step s0 = kbase / 128 of the panel on (kbase is a
            // multiple of 128 whenever B is packed)
            const int64_t panel = n0 / kPanelRows, prow = n0 % kPanelRows, s0 = kbase / 128;
            const uint8_t *bt = p.b_q + ((g * p.NP + panel) * p.KS + s0) * kTileBytes + prow * 128;
            rb = make_srd(bt, (uint32_t)((int64_t)(p.KS - s0) * kTileBytes - prow * 128));
            const uint8_t *bs = p.b_s + ((g * p.NP + panel) * p.KS + s0) * kScaleStepBytes + (prow / 16) * 64;
            rsb = make_srd(bs, (uint32_t)((int64_t)(p.KS - s0) * kScaleStepBytes - (prow / 16) * 64));
            rsb_c = make_rsrc(p.b_s, 0u);
        } else {
            const int64_t rows_b = min((int64_t)BN, N - n0);
            const uint32_t b_bytes = (uint32_t)((rows_b - 1) * p.ldb + K);
            const uint32_t bs_bytes = (uint32_t)((rows_b - 1) * p.lsb + KB);
            rb = make_srd(p.b_q + n0 * p.ldb + kbase, b_bytes);
            rsb = make_srd(p.b_s + n0 * p.lsb + kbase / 32, bs_bytes);
            rsb_c = make_rsrc(p.b_s + n0 * p.lsb + kbase / 32, bs_bytes);
        }
    }

    // APACK: offset of this lane's 16 bytes of the tile's 8-row segment seg at
    // k-step ks (segments past the tile's rows read zeros: in a grouped tile
    // the panel rows past the group are another group's)
    __device__ __forceinline__ uint32_t apack_off(int ks, int seg) const {
        const int row = a_r0 + seg * 8;
        return seg * 8 < rows_a ? ((uint32_t)((row >> 8) * KSa + ks) * (uint32_t)kTileBytes +
                                   (uint32_t)((row & 255) * 128 + lane * 16))
                                : kOOB;
    }
    // APACK: this lane's dword of the scale records of atoms 4q .. 4q + 3
    // (lane l: atom 4q + l / 16, dword l % 16 of its 64-byte record)
    __device__ __forceinline__ uint32_t apack_scale_off(int ks, int q) const {
        const int a = q * 4 + (lane >> 4), row = a_r0 + a * 16;
        return a * 16 < rows_a ? ((uint32_t)((row >> 8) * KSa + ks) * (uint32_t)kScaleStepBytes +
                                  (uint32_t)(((row & 255) >> 4) * 64 + (lane & 15) * 4))
                               : kOOB;
    }

    // global -> LDS copies of k-step ks into stage st (this wave's share)
    __device__ __forceinline__ void issue(int ks, int st) const { issue_at(ks, lds0 + st * STAGE); }
    // The copies of a 256-row tile with the two-stage ring are issued by
    // waves 0-3 only (one per SIMD; waves w and w + 4 share a SIMD): issuing
    // a step's 48-64 KB of copies stalls the issuing wave for ~1300-1900
    // clocks while the address unit drains, and this way the other wave of
    // each SIMD starts its MFMAs at once instead of both stalling.
    // Measured (MI355X, 8192x24576x4096 / 8192x4096x12288): 746 -> 716 us
    // and 367 -> 353 us, bit-identical.  (Even waves as copiers, i.e. both
    // waves of two SIMDs: slower.)  Three-stage rings keep every wave's
    // share, since their waits count each wave's own copies.
    static constexpr bool kCopiers = BM == 256 && (BN == 256 || BN == 128);
    __device__ __forceinline__ void issue_copiers(int ks, uint32_t sbase) const {
        if (w >= 4) return;
        const int cw = w;
#pragma unroll
        for (int i = 0; i < BM / 32; ++i) {
            const int seg = i * 4 + cw;
            uint32_t off;
            if constexpr (APACK) off = apack_off(ks, seg);
            else {
                const int rr = seg * 8 + (lane >> 3);
                const int c = (lane & 7) ^ (int)swz((uint32_t)rr);
                const int kk = ks * 128 + c * 16;
                off = kk < Ki ? (uint32_t)(rr * lda + kk) : kOOB;
            }
            dma16(ra, off, sbase + seg * 1024);
        }
#pragma unroll
        for (int i = 0; i < BN / 32; ++i) {
            const int seg = i * 4 + cw;
            uint32_t off;
            if constexpr (BPACK) {
                off = (uint32_t)ks * (uint32_t)kTileBytes + seg * 1024 + lane * 16;
            } else {
                const int rr = seg * 8 + (lane >> 3);
                const int c = (lane & 7) ^ (int)swz((uint32_t)rr);
                const int kk = ks * 128 + c * 16;
                off = kk < Ki ? (uint32_t)(rr * ldb + kk) : kOOB;
            }
            dma16(rb, off, sbase + BM * 128 + seg * 1024);
        }
        if constexpr (APACK) dma4(rsa, apack_scale_off(ks, cw), sbase + SA_OFF + cw * 256);
        else if constexpr (SA_LDS) dma4(rsa, (uint32_t)((cw * 64 + lane) * lsa + ks * 4), sbase + SA_OFF + cw * 256);
        if constexpr (SB_LDS) {
            if (cw < BN / 64) {
                uint32_t off;
                if constexpr (BPACK) off = (uint32_t)(ks * kScaleStepBytes + cw * 256 + lane * 4);
                else off = (uint32_t)((cw * 64 + lane) * lsb + ks * 4);
                dma4(rsb, off, sbase + SB_OFF + cw * 256);
            }
        }
    }
    // copies of a step for the two-stage rings (whose waits are vmcnt(0))
    __device__ __forceinline__ void issue2(int ks, uint32_t sbase) const {
        if constexpr (kCopiers) issue_copiers(ks, sbase);
        else issue_at(ks, sbase);
    }
    // the same into the stage at LDS byte address sbase, each wave its share
    __device__ __forceinline__ void issue_at(int ks, uint32_t sbase) const {
#pragma unroll
        for (int i = 0; i < BM / (8 * kWaves); ++i) {
            const int seg = i * kWaves + w;            // 1 KB LDS segment = 8 rows
            uint32_t off;
            if constexpr (APACK) off = apack_off(ks, seg);
            else {
                const int rr = seg * 8 + (lane >> 3);
                const int c = (lane & 7) ^ (int)swz((uint32_t)rr);
                const int kk = ks * 128 + c * 16;
                off = kk < Ki ? (uint32_t)(rr * lda + kk) : kOOB;
            }
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
                off = kk < Ki ? (uint32_t)(rr * ldb + kk) : kOOB;
            }
            dma16(rb, off, sbase + BM * 128 + seg * 1024);
        }
        // scale copies: 256 B segments, one per wave that owns one
        if constexpr (SA_LDS) {
            if (w < BM / 64) {
                const int rr = w * 64 + lane;
                if constexpr (APACK) dma4(rsa, apack_scale_off(ks, w), sbase + SA_OFF + w * 256);
                else dma4(rsa, (uint32_t)(rr * lsa + ks * 4), sbase + SA_OFF + w * 256);
            }
        }
        if constexpr (SB_LDS) {
            if (w < BN / 64) {
                uint32_t off;
                if constexpr (BPACK) off = (uint32_t)(ks * kScaleStepBytes + w * 256 + lane * 4);
                else off = (uint32_t)((w * 64 + lane) * lsb + ks * 4);
                dma4(rsb, off, sbase + SB_OFF + w * 256);
            }
        }
    }

    // K % 128 != 0: scale bytes by compiler-visible loads (K tail reads 0)
    __device__ __forceinline__ void fetch_sa(int ks, uint32_t *dst) const {
        const int blk = ks * 4 + lblk;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int rr = wm * WTM + i * 16 + lrow;
            const uint32_t off = blk < KBi ? (uint32_t)(rr * lsa + blk) : kOOB;
            dst[i] = __builtin_amdgcn_raw_buffer_load_b8(rsa_c, off, 0, 0);
        }
    }
    __device__ __forceinline__ void fetch_sb(int ks, uint32_t *dst) const {
        const int blk = ks * 4 + lblk;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int rr = wn * WTN + j * 16 + lrow;
            const uint32_t off = blk < KBi ? (uint32_t)(rr * lsb + blk) : kOOB;
            dst[j] = __builtin_amdgcn_raw_buffer_load_b8(rsb_c, off, 0, 0);
        }
    }

    // SAC: A scale bytes of k-steps [8c, 8c + 8) of every tile row, 32 bytes
    // per row, into the chunk buffer at LDS address cbase: two lanes per row,
    // 16 bytes each, each wave a 32-row share; row r's 16-byte half h sits at
    // r * 32 + 16 * (h ^ (r / 8 % 2)) so that the byte reads of 16
    // consecutive rows (one per lane) fall in distinct banks.  Rows past the
    // operand's end read zero; bytes past a row's K range are never read.
    __device__ __forceinline__ void issue_sa_chunk(int c, uint32_t cbase) const {
        static_assert(BM == 8 * 32, "eight waves of 32 rows");
        const int rr = w * 32 + (lane >> 1), h = (lane & 1) ^ ((rr >> 3) & 1);
        dma16(rsa, (uint32_t)(rr * lsa + c * 32 + h * 16), cbase + w * 1024);
    }
    // SBC: the same for the canonical B tile's scales
    __device__ __forceinline__ void issue_sb_chunk(int c, uint32_t cbase) const {
        static_assert(BN == 8 * 32, "eight waves of 32 rows");
        const int rr = w * 32 + (lane >> 1), h = (lane & 1) ^ ((rr >> 3) & 1);
        dma16(rsb, (uint32_t)(rr * lsb + c * 32 + h * 16), cbase + w * 1024);
    }
    // byte kb (0..31) of row r in a chunk buffer
    __device__ __forceinline__ static int chunk_byte(int r, int kb) {
        return r * 32 + (((kb >> 4) ^ ((r >> 3) & 1)) << 4) + (kb & 15);
    }

    // scale bytes of one step from LDS (the MFMA reads bits [7:0], op_sel 0);
    // chunk: the SAC chunk buffer holding step ks
    __device__ __forceinline__ void lds_scales(const uint8_t *st, int *sas, int *sbs, const uint8_t *chunk = nullptr,
                                               int ks = 0, const uint8_t *chunk_b = nullptr) const {
        if constexpr (SBC) {
            const int kb = (ks % kChunkSteps) * 4 + lblk;
#pragma unroll
            for (int j = 0; j < FN; ++j) sbs[j] = chunk_b[chunk_byte(wn * WTN + j * 16 + lrow, kb)];
        }
        if constexpr (APACK) {
#pragma unroll
            for (int i = 0; i < FM; ++i) sas[i] = st[SA_OFF + (wm * FM + i) * 64 + lane];
        } else if constexpr (SA_LDS) {
#pragma unroll
            for (int i = 0; i < FM; ++i) sas[i] = st[SA_OFF + (wm * WTM + i * 16 + lrow) * 4 + lblk];
        }
        if constexpr (SAC) {
            const int kb = (ks % kChunkSteps) * 4 + lblk;
#pragma unroll
            for (int i = 0; i < FM; ++i) sas[i] = chunk[chunk_byte(wm * WTM + i * 16 + lrow, kb)];
        }
        if constexpr (SB_LDS) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (BPACK) sbs[j] = st[SB_OFF + (wn * FN + j) * 64 + lane];
                else sbs[j] = st[SB_OFF + (wn * WTN + j * 16 + lrow) * 4 + lblk];
            }
        }
    }

    __device__ __forceinline__ void lds_bfrags(const uint8_t *st, v8i *bf) const {
        const uint8_t *sb = st + BM * 128 + wn * WTN * 128;
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = lds_frag(sb + j * 16 * 128, lane);
    }

    // MFMAs of A rows [i0, i1) of one step against the B fragments in
    // registers.  The B fragment is the first operand, so each 16x16 result
    // is C^T: lane l accumulates C[16i + l % 16][16j + 4 (l / 16) + r],
    // r = 0..3 -- four consecutive columns of one row, which the epilogue
    // moves as one 8-byte (bf16) or 16-byte (fp32) piece.
    __device__ __forceinline__ void mma_rows(const uint8_t *st, int i0, int i1, const v8i *bf, const int *sas,
                             const int *sbs, v4f (*acc)[FN]) const {
        const uint8_t *sa = st + wm * WTM * 128;
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            const v8i af = lds_frag(sa + i * 16 * 128, lane);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bf[j], af, acc[i][j], 0, 0, 0, sbs[j], 0, sas[i]);
        }
    }

    // ---- accurate path (mxfp8_gemm_accurate): BF16 MFMA on operands
    // converted exactly.  Every E4M3 element times its block's scale is a
    // 4-bit significand with an exponent inside BF16's range whenever the
    // scale code lies in [3, 246], so the conversion is exact, every product
    // of two such BF16 values is exact in fp32, and the BF16 matrix
    // instruction adds them with fp32 accuracy (measured: at most 2^-20 of
    // the largest product), far inside 1e-4 * sum|ab|.

    // The four block scales of step ks (byte t: block 4 ks + t) of the
    // lane's row in A atom i and B atom j.  Rows outside the operands and
    // blocks past K (whose elements are all zero) read as 127, whatever the
    // layout stores there, so packed and canonical B take the same path.
    __device__ __forceinline__ void acc_scales(const uint8_t *st, int ks, const uint8_t *chunk,
                                               const uint8_t *chunk_b, uint32_t *sa4, uint32_t *sb4) const {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = wm * WTM + i * 16 + lrow;
            if constexpr (SA_LDS) {
                sa4[i] = *reinterpret_cast<const uint32_t *>(st + SA_OFF + r * 4);
            } else if constexpr (SAC) {
                sa4[i] = *reinterpret_cast<const uint32_t *>(chunk + chunk_byte(r, (ks % kChunkSteps) * 4));
            } else {
                uint32_t v = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int blk = ks * 4 + t;
                    const uint32_t off = blk < KBi ? (uint32_t)(r * lsa + blk) : kOOB;
                    v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsa_c, off, 0, 0) << (8 * t);
                }
                sa4[i] = v;
            }
            sa4[i] = neutral_outside(sa4[i], r < rows_a, ks);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int r = wn * WTN + j * 16 + lrow;
            if constexpr (BPACK) {
                const uint8_t *p = st + SB_OFF + (wn * FN + j) * 64 + lrow;
                sb4[j] = (uint32_t)p[0] | ((uint32_t)p[16] << 8) | ((uint32_t)p[32] << 16) | ((uint32_t)p[48] << 24);
            } else if constexpr (SBC) {
                sb4[j] = *reinterpret_cast<const uint32_t *>(chunk_b + chunk_byte(r, (ks % kChunkSteps) * 4));
            } else if constexpr (SB_LDS) {
                sb4[j] = *reinterpret_cast<const uint32_t *>(st + SB_OFF + r * 4);
            } else {
                uint32_t v = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int blk = ks * 4 + t;
                    const uint32_t off = blk < KBi ? (uint32_t)(r * lsb + blk) : kOOB;
                    v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsb_c, off, 0, 0) << (8 * t);
                }
                sb4[j] = v;
            }
            sb4[j] = neutral_outside(sb4[j], r < rows_b, ks);
        }
    }

    // 127 in every byte of a row outside the operand, and in the bytes of
    // blocks at or past K/32
    __device__ __forceinline__ uint32_t neutral_outside(uint32_t v, bool row_in, int ks) const {
        if (!row_in) return 0x7F7F7F7Fu;
        const int valid = KBi - ks * 4;                 // blocks of this step inside K
        if (valid >= 4) return v;
        const uint32_t keep = valid <= 0 ? 0u : (1u << (8 * valid)) - 1u;
        return (v & keep) | (0x7F7F7F7Fu & ~keep);
    }

    // 8 E4M3 bytes of the lane's row of a 16-row atom: K = 32 t + 8 (lane / 16)
    // .. + 7 of the step (the K slice a lane supplies to the 16x16x32 BF16
    // MFMA), from the swizzled 128-byte LDS rows
    __device__ __forceinline__ v2i lds_k8(const uint8_t *atom, int t) const {
        const int g = lane >> 4;
        const int c = 2 * t + (g >> 1);
        return *reinterpret_cast<const v2i *>(atom + lrow * 128 + (int)((c ^ (int)swz((uint32_t)lrow)) * 16) +
                                              (g & 1) * 8);
    }

    // the BF16 fragment of those 8 elements times 2^(code - 127)
    __device__ __forceinline__ static v8bf cvt8(v2i v, uint32_t code) {
        const float s = code == 0 ? bits_to_float(0x00400000u) : bits_to_float(code << 23);
        const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.x, s, false);
        const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.x, s, true);
        const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.y, s, false);
        const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v.y, s, true);
        return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    }

    // true if every scale byte of the step lies in [3, 246] (exact folded
    // conversion), the same in every lane of the wave
    __device__ __forceinline__ static bool scales_foldable(const uint32_t *sa4, const uint32_t *sb4) {
        uint32_t bad = 0;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t c = (sa4[i] >> (8 * t)) & 0xFFu;
                bad |= (uint32_t)(c < 3u || c > 246u);
            }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t c = (sb4[j] >> (8 * t)) & 0xFFu;
                bad |= (uint32_t)(c < 3u || c > 246u);
            }
        return __ballot(bad != 0) == 0;
    }

    // One k-step on the accurate path.  Folded: the scales ride the
    // conversions and the four 32-K MFMAs per tile accumulate straight into
    // acc.  Otherwise (a scale outside [3, 246] somewhere in the wave's
    // operands): unscaled BF16 products per block, each block's 16x16 sum
    // scaled by 2^(sa + sb - 254) with ldexp and added in fp32.
    __device__ __forceinline__ void acc_step(const uint8_t *st, int ks, const uint8_t *chunk,
                                             const uint8_t *chunk_b, v4f (*acc)[FN]) const {
        uint32_t sa4[FM], sb4[FN];
        acc_scales(st, ks, chunk, chunk_b, sa4, sb4);
        const uint8_t *sa = st + wm * WTM * 128;
        const uint8_t *sb = st + BM * 128 + wn * WTN * 128;
        if (scales_foldable(sa4, sb4)) {
            // Folded: every element carries its own scale, so the K slots of
            // the four 16x16x32 MFMAs may be any split of the step's 128 K
            // that A and B share.  The lane's 32-byte fragment of the scaled
            // FP8 MFMA (K 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15,
            // g = lane / 16; conflict-free 16-byte LDS reads) is cut into
            // four 8-byte slices, slice v feeding MFMA v; slices 0-1 belong
            // to block g / 2, slices 2-3 to block 2 + g / 2.
            const int b0 = lblk >> 1, b1 = 2 + (lblk >> 1);
            v8bf bf[FN][4];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const v8i f = lds_frag(sb + j * 16 * 128, lane);
                const uint32_t c0 = (sb4[j] >> (8 * b0)) & 0xFFu, c1 = (sb4[j] >> (8 * b1)) & 0xFFu;
                bf[j][0] = cvt8(v2i{f[0], f[1]}, c0);
                bf[j][1] = cvt8(v2i{f[2], f[3]}, c0);
                bf[j][2] = cvt8(v2i{f[4], f[5]}, c1);
                bf[j][3] = cvt8(v2i{f[6], f[7]}, c1);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v8i f = lds_frag(sa + i * 16 * 128, lane);
                const uint32_t c0 = (sa4[i] >> (8 * b0)) & 0xFFu, c1 = (sa4[i] >> (8 * b1)) & 0xFFu;
                const v8bf af[4] = {cvt8(v2i{f[0], f[1]}, c0), cvt8(v2i{f[2], f[3]}, c0),
                                    cvt8(v2i{f[4], f[5]}, c1), cvt8(v2i{f[6], f[7]}, c1)};
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j][v], af[v], acc[i][j], 0, 0, 0);
            }
            return;
        }
        // lane l holds C[row l % 16][cols 4 (l / 16) + r]: the column scales
        // are the B scale words of lanes 4 (l / 16) + r
        uint32_t sbc[FN][4];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) sbc[j][r] = (uint32_t)__shfl((int)sb4[j], 4 * (lane >> 4) + r);
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v8bf bf[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = cvt8(lds_k8(sb + j * 16 * 128, t), 127u);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v8bf af = cvt8(lds_k8(sa + i * 16 * 128, t), 127u);
                const int ca = (int)((sa4[i] >> (8 * t)) & 0xFFu);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const v4f p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af, zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int cb = (int)((sbc[j][r] >> (8 * t)) & 0xFFu);
                        float v = __builtin_ldexpf(p[r], ca + cb - 254);
                        if (ca == 255 || cb == 255) v = __builtin_nanf("");
                        acc[i][j][r] += v;
                    }
                }
            }
        }
    }
};

template <int V>
struct IntC {
    static constexpr int value = V;
};

__device__ __forceinline__ void wait_copies_and_sync() {
    // every copy this wave issued has landed (vmcnt; a builtin, so the
    // compiler knows it too), then every wave's (barrier)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
}

// Tile coordinates of this workgroup; false if it has no tile.
template <int BM, int BN, bool GROUPED>
__device__ __forceinline__ bool tile_of(const GemmParams &p, int64_t &m0, int64_t &m_end, int64_t &n0, int64_t &g) {
    int tm, tn;
    if constexpr (GROUPED) {
        // the grid covers the worst case (every group's last tile partial);
        // renumber over the tiles that exist so that each XCD gets an equal
        // contiguous share and the spare workgroups (highest ids) exit
        const int tiles_m = count_group_tiles<BM>(p.offsets, p.G, p.M, threadIdx.x & 63);
        const int n = tiles_m * p.tiles_n;
        if ((int)blockIdx.x >= n) return false;
        grouped_order(xcd_logical(blockIdx.x, n), tiles_m, p.tiles_n, tm, tn);
    } else {
        grouped_order(xcd_logical(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
    }
    if (tm >= p.tiles_m || tn >= p.tiles_n) return false;
    g = 0;
    if constexpr (GROUPED) {
        int64_t lo, hi;
        int tig;
        const int gg = find_group<BM>(p.offsets, p.G, p.M, tm, threadIdx.x & 63, lo, hi, tig);
        if (gg < 0) return false;
        g = gg;
        m0 = lo + (int64_t)tig * BM;
        m_end = hi;
    } else {
        m0 = (int64_t)tm * BM;
        m_end = p.M;
    }
    n0 = (int64_t)tn * BN;
    return true;
}

// Grouped-K mode: tile -> (group g, tile row, tile column); the group's K range
// is its token range [o_g, o_g+1) of the operands' rows (clamped like
// find_group, so a malformed table can only drop work).  False past the end.
// Tiles are taken in dispatch order, not renumbered per XCD: group sizes are
// skewed (a few experts hold most tokens), and an XCD-contiguous range would
// put a heavy group's long tiles all on one XCD.  In dispatch order each
// group's tiles are dealt round-robin over the XCDs (measured on a Zipf(1.1)
// routing of 8192 tokens: 1449 -> 636 us for the gate_up weight gradient).
template <int BM, int BN>
__device__ __forceinline__ bool tile_of_gk(const GemmParams &p, int64_t &m0, int64_t &m_end, int64_t &n0,
                                           int64_t &g, int64_t &kbase, int64_t &kbound) {
    const int per = p.tiles_m * p.tiles_n;
    const int L = blockIdx.x;
    g = L / per;
    if (g >= p.G) return false;
    int tm, tn;
    grouped_order(L % per, p.tiles_m, p.tiles_n, tm, tn);
    int64_t lo = p.offsets[g], hi = p.offsets[g + 1];
    lo = lo < 0 ? 0 : (lo > p.K ? p.K : lo);
    hi = hi < lo ? lo : (hi > p.K ? p.K : hi);
    kbase = lo;
    kbound = hi - lo;
    m0 = (int64_t)tm * BM;
    m_end = p.M;
    n0 = (int64_t)tn * BN;
    return true;
}

// C store, element by element: lane holds C[lane % 16][4*(lane/16) + r] of
// each 16x16 tile (C^T fragments; used for blocks that cross the matrix edge).
template <int FM, int FN, bool OUT_BF16>
__device__ __forceinline__ void store_tile_scalar(const GemmParams &p, int64_t row0, int64_t col0, int64_t m_end,
                                  v4f (*acc)[FN], int lane) {
    const int64_t N = p.N;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t row = row0 + i * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t col = col0 + j * 16 + (lane >> 4) * 4 + r;
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

// C store through LDS: each wave writes its block into its own LDS region in
// row-major order (rows padded by 16 B against bank conflicts), then reads it
// back 16 bytes per lane so every global store is a whole 16-byte piece of a
// contiguous row segment.  Rows go in passes of PR so the regions of all
// waves fit the LDS the main loop used.  Callers sync before (the stages are
// reused) and use this only for tiles whose columns are inside C with
// 16-byte aligned rows; rows at or past m_end are not written.
//
// The stores are buffer stores over this wave's rows of C that exist (rows
// at or past m_end fall outside the descriptor and are dropped), so every
// wave issues exactly store_tile_lds_count() of them whatever m_end is, and
// a caller may wait for VMEM operations issued before them with
// vmcnt(count) (vector memory operations complete in issue order), leaving
// the stores to drain behind its next work.  Returns false (pointer stores,
// count not exact) when the wave's block spans 4 GiB or more of C.
// Cache policy of C stores of whole 128-byte rows (sc0 | nt: streamed, not
// kept in the L2 that holds the operands).  Measured against the default
// policy: gemm_ws_kernel qkv 88.4 -> 85.2 us, 2048x4096x4096 33.7 -> 28.6 us;
// the grouped MoE launches gate_up 268 -> 262 us, down 176 -> 166 us; the
// MLP GEMMs 0-3% faster; the paired launch 2.5% slower, so it keeps the
// default.  (Streamed stores of half rows wrote 1.5x the bytes of C.)
constexpr int kStoreStream = 3;

template <int FM, int FN, bool OUT_BF16, int LDS_BYTES, int NW = kWaves>
struct EpilogueShape {
    static constexpr int ES = OUT_BF16 ? 2 : 4;
    static constexpr int WTM = FM * 16, WTN = FN * 16;
    static constexpr int ROWB = WTN * ES + 16;                       // padded LDS row
    static constexpr int PR0 = LDS_BYTES / (NW * ROWB);              // rows per pass that fit
    static constexpr int PR = PR0 >= WTM ? WTM : (PR0 >= 64 ? 64 : (PR0 >= 32 ? 32 : 16));
    static_assert(PR >= 16 && WTM % PR == 0 && NW * PR * ROWB <= LDS_BYTES, "epilogue LDS");
    static constexpr int LPR = WTN * ES / 16;                         // lanes per row (16 B each)
    static constexpr int RPI = 64 / LPR;                              // rows per store instruction
    static constexpr int kStores = WTM / RPI;                         // store instructions per wave
};
template <int FM, int FN, bool OUT_BF16, int LDS_BYTES, int NW = kWaves, int POL = kStoreStream>
__device__ __forceinline__ bool store_tile_lds(const GemmParams &p, int64_t row0, int64_t col0, int64_t m_end,
                               v4f (*acc)[FN], int lane, int w, uint8_t *smem) {
    using E = EpilogueShape<FM, FN, OUT_BF16, LDS_BYTES, NW>;
    constexpr int ES = E::ES, WTN = E::WTN, WTM = E::WTM, ROWB = E::ROWB, PR = E::PR, LPR = E::LPR,
                  RPI = E::RPI;
    uint8_t *cw = smem + w * PR * ROWB;
    const int64_t N = p.N;
    const bool counted = (int64_t)WTM * N * ES <= 0xFFFFFFFFll;
    const int64_t rows_here = m_end - row0;
    const uint32_t range = rows_here <= 0 ? 0u
                           : (uint32_t)((min(rows_here, (int64_t)WTM) - 1) * N * ES + WTN * ES);
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(static_cast<uint8_t *>(p.c) + (rows_here > 0 ? (row0 * N + col0) * ES : 0), range);
#pragma unroll
    for (int pass = 0; pass < WTM / PR; ++pass) {
        // scatter this pass's rows (16-row MFMA tiles i in [pass*PR/16, ...)):
        // each lane's four consecutive columns of one row as one LDS write
#pragma unroll
        for (int i = pass * (PR / 16); i < (pass + 1) * (PR / 16); ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int rl = (i - pass * (PR / 16)) * 16 + (lane & 15);
                const int cl = j * 16 + (lane >> 4) * 4;
                if constexpr (OUT_BF16) {
                    const uint32_t lo = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
                    const uint32_t hi = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
                    *reinterpret_cast<v2i *>(cw + rl * ROWB + cl * 2) = v2i{(int)lo, (int)hi};
                } else {
                    *reinterpret_cast<v4f *>(cw + rl * ROWB + cl * 4) = acc[i][j];
                }
            }
        }
        // gather 16 B per lane and store whole row segments
#pragma unroll
        for (int r0 = 0; r0 < PR; r0 += RPI) {
            const int rl = r0 + lane / LPR;
            const int cb = (lane % LPR) * 16;
            const v4i v = *reinterpret_cast<const v4i *>(cw + rl * ROWB + cb);
            if (counted) {
                const uint32_t off = (uint32_t)(pass * PR + rl) * (uint32_t)(N * ES) + (uint32_t)cb;
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, (int)off, 0, POL);
            } else {
                const int64_t row = row0 + pass * PR + rl;
                uint8_t *dst = static_cast<uint8_t *>(p.c) + (row * N + col0) * ES + cb;
                if (row < m_end) *reinterpret_cast<v4i *>(dst) = v;
            }
        }
    }
    return counted;
}

// ---------------------------------------------------------------- 2 stages
// One barrier at the top of each step; copies of step k+1 overlap step k.
// GK (grouped-K, weight gradients of the experts): C_g = A[:, K_g] B[:, K_g]^T
// for every group g, K_g its token range, C_g at c + g * c_stride.
// Copy instructions one wave issues per k-step (KALIGN: tiles and both scale
// sets through LDS): its tile segments plus one scale copy per 64 rows it owns.
template <int BM, int BN>
__device__ __forceinline__ int copies_per_step(int w) {
    return BM / (8 * kWaves) + BN / (8 * kWaves) + (w < BM / 64 ? 1 : 0) + (w < BN / 64 ? 1 : 0);
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [N0, N0 + 2]
template <int N0>
__device__ __forceinline__ void wait_vm_upto(int n) {
    if (n <= N0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(N0));
    else if (n == N0 + 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(N0 + 1));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(N0 + 2));
}

// One BM x BN tile of C: k-loop over [kbase, kbase + kbound) of every row
// (KS k-steps) and the store.  smem holds NST stages.
// NST stages: the copies of step ks+NST-1 are issued at the top of step ks.
// NST = 3 needs every copy to go through LDS (KALIGN) so that a wave's copy
// count per step is fixed and the wait can leave the next steps in flight.
template <int BM, int BN, int WM, bool BPACK, bool OUT_BF16, bool KALIGN, int NST, bool SAC = false,
          bool ACC = false, bool APACK = false>
__device__ __forceinline__ void gemm_tile(GemmParams &p, int64_t m0, int64_t m_end, int64_t n0, int64_t g,
                                          int64_t kbase, int64_t kbound, int KS, uint8_t *smem) {
    using T = TileOps<BM, BN, WM, BPACK, KALIGN, SAC, APACK>;
    static_assert(!(APACK && ACC), "packed A on the fast path only");
    static_assert(!SAC || NST == 2, "chunked A scales with the two-stage ring");
    // SAC chunk buffers (two) after the stage ring, then (SBC) two for B
    uint8_t *chunks = smem + NST * T::STAGE;
    uint8_t *chunks_b = chunks + 2 * T::CHUNK;
    constexpr int FM = T::FM, FN = T::FN;
    static_assert(NST == 2 || (NST == 3 && KALIGN), "three stages need all copies through LDS");
    T t;
    t.init(p, m0, m_end, n0, g, smem, kbase, kbound);

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint32_t sa_cur[FM], sa_nxt[FM], sb_cur[FN], sb_nxt[FN];
    if (KS > 0) {                       // an empty group (grouped-K) stores zeros
        if constexpr (SAC) t.issue_sa_chunk(0, t.lds0 + NST * T::STAGE);
        if constexpr (T::SBC) t.issue_sb_chunk(0, t.lds0 + NST * T::STAGE + 2 * T::CHUNK);
        if constexpr (T::SA_REG && !ACC) t.fetch_sa(0, sa_nxt);
        if constexpr (T::SB_REG && !ACC) t.fetch_sb(0, sb_nxt);
        if constexpr (NST == 2) t.issue2(0, t.lds0);
        else t.issue(0, 0);
        if constexpr (NST == 3) {
            if (KS > 1) t.issue(1, 1);
        }
    }
    const int ncopies = copies_per_step<BM, BN>(t.w);

    int cur = 0;
    for (int ks = 0; ks < KS; ++ks) {
        if constexpr (NST == 3) {
            // this wave's copies of step ks have landed: only those of step
            // ks+1 (issued after them, if any) may still be in flight
            if (ks + 1 < KS) wait_vm_upto<BM / (8 * kWaves) + BN / (8 * kWaves)>(ncopies);
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __syncthreads();
        } else {
            wait_copies_and_sync();
        }
        if constexpr (SAC) {
            // at the first step of chunk c every wave is past chunk c-1's
            // steps: its buffer takes chunk c+1 (awaited at the next step's
            // top with everything else)
            const int c = ks / T::kChunkSteps;
            if (ks % T::kChunkSteps == 0 && (c + 1) * T::kChunkSteps < KS) {
                t.issue_sa_chunk(c + 1, t.lds0 + NST * T::STAGE + ((c + 1) & 1) * T::CHUNK);
                if constexpr (T::SBC)
                    t.issue_sb_chunk(c + 1, t.lds0 + NST * T::STAGE + 2 * T::CHUNK + ((c + 1) & 1) * T::CHUNK_B);
            }
        }
        if constexpr (T::SA_REG && !ACC) {
#pragma unroll
            for (int i = 0; i < FM; ++i) sa_cur[i] = sa_nxt[i];
            if (ks + 1 < KS) t.fetch_sa(ks + 1, sa_nxt);
        }
        if constexpr (T::SB_REG && !ACC) {
#pragma unroll
            for (int j = 0; j < FN; ++j) sb_cur[j] = sb_nxt[j];
            if (ks + 1 < KS) t.fetch_sb(ks + 1, sb_nxt);
        }
        if constexpr (NST == 3) {
            // stage (cur + 2) % 3 held step ks-1, which every wave finished
            // before the barrier above
            if (ks + 2 < KS) t.issue(ks + 2, cur == 0 ? 2 : cur - 1);
        } else {
            if (ks + 1 < KS) t.issue2(ks + 1, t.lds0 + (cur ^ 1) * T::STAGE);
        }

        const uint8_t *st = smem + cur * T::STAGE;
        if constexpr (ACC) {
            t.acc_step(st, ks, chunks + ((ks / T::kChunkSteps) & 1) * T::CHUNK,
                       chunks_b + ((ks / T::kChunkSteps) & 1) * T::CHUNK_B, acc);
            cur = cur + 1 == NST ? 0 : cur + 1;
            continue;
        }
        int sas[FM], sbs[FN];
        t.lds_scales(st, sas, sbs, chunks + ((ks / T::kChunkSteps) & 1) * T::CHUNK, ks,
                     chunks_b + ((ks / T::kChunkSteps) & 1) * T::CHUNK_B);
        if constexpr (T::SA_REG) {
#pragma unroll
            for (int i = 0; i < FM; ++i) sas[i] = (int)(sa_cur[i] & 0xFFu);
        }
        if constexpr (T::SB_REG) {
#pragma unroll
            for (int j = 0; j < FN; ++j) sbs[j] = (int)(sb_cur[j] & 0xFFu);
        }
        v8i bf[FN];
        t.lds_bfrags(st, bf);
        t.mma_rows(st, 0, FM, bf, sas, sbs, acc);
        cur = cur + 1 == NST ? 0 : cur + 1;
    }
    (void)ncopies;
    (void)chunks;
    (void)chunks_b;
    const int64_t row0 = m0 + t.wm * T::WTM, col0 = n0 + t.wn * T::WTN;
    constexpr int ES = OUT_BF16 ? 2 : 4;
    // uniform over the workgroup: the tile's columns inside C, rows 16 B
    // aligned (partial row ranges, e.g. the last tile of an expert, are masked)
    const bool inside = n0 + BN <= p.N && (p.N * ES) % 16 == 0;
    if (inside) {
        __syncthreads();                    // every wave is done with the stages
        store_tile_lds<FM, FN, OUT_BF16, NST * T::STAGE>(p, row0, col0, m_end, acc, t.lane, t.w, smem);
    } else {
        store_tile_scalar<FM, FN, OUT_BF16>(p, row0, col0, m_end, acc, t.lane);
    }
}

template <int BM, int BN, int WM, bool BPACK, bool OUT_BF16, bool GROUPED, bool KALIGN, bool GK = false,
          int NST = 2, bool SAC = false, bool ACC = false, bool APACK = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
    using T = TileOps<BM, BN, WM, BPACK, KALIGN, SAC, APACK>;
    constexpr int LDS = NST * T::STAGE + (SAC ? 2 * T::CHUNK + 2 * T::CHUNK_B : 0);
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(!GK || (!BPACK && !KALIGN && !GROUPED), "grouped-K reads canonical operands");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
    int64_t m0, m_end, n0, g, kbase = 0, kbound = -1;
    int KS = p.KS;
    if constexpr (GK) {
        if (!tile_of_gk<BM, BN>(p, m0, m_end, n0, g, kbase, kbound)) return;
        KS = (int)((kbound + 127) / 128);
        p.c = static_cast<uint8_t *>(p.c) + g * p.c_stride * (OUT_BF16 ? 2 : 4);
    } else {
        if (!tile_of<BM, BN, GROUPED>(p, m0, m_end, n0, g)) return;
    }
    gemm_tile<BM, BN, WM, BPACK, OUT_BF16, KALIGN, NST, SAC, ACC, APACK>(p, m0, m_end, n0, g, kbase, kbound, KS,
                                                                          smem);
}

// Grouped-K (expert weight gradients) with T % 128 == 0: a tile whose token
// range starts and ends on a multiple of 128 (one k-step) takes the aligned
// path, its scale dwords copied through LDS with the tiles; any other tile
// reads its scale bytes through registers as gemm_kernel<..., GK> does.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void gemm_gk_aligned_kernel(GemmParams p) {
    constexpr int SA = 2 * TileOps<256, 256, 2, false, true>::STAGE;
    constexpr int SU = 2 * TileOps<256, 256, 2, false, false>::STAGE;
    static_assert(SA <= 160 * 1024 && SU <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SA > SU ? SA : SU];
    int64_t m0, m_end, n0, g, kbase, kbound;
    if (!tile_of_gk<256, 256>(p, m0, m_end, n0, g, kbase, kbound)) return;
    const int KS = (int)((kbound + 127) / 128);
    p.c = static_cast<uint8_t *>(p.c) + g * p.c_stride * (OUT_BF16 ? 2 : 4);
    if ((kbase & 127) == 0 && (kbound & 127) == 0)
        gemm_tile<256, 256, 2, false, OUT_BF16, true, 2>(p, m0, m_end, n0, g, kbase, kbound, KS, smem);
    else
        gemm_tile<256, 256, 2, false, OUT_BF16, false, 2>(p, m0, m_end, n0, g, kbase, kbound, KS, smem);
}

// Split-K (few output tiles): workgroup -> (slice s, tile); slice s covers
// k-steps [s * split_steps, (s+1) * split_steps) and writes its fp32 partial
// tile to p.c + s * c_stride (c_stride = M * N rounded up to 4 floats).  A slice ending before K % 128 (only the last,
// when K % 128 != 0) takes the byte-scale path, the others the aligned one.
template <bool BPACK>
__global__ __launch_bounds__(kThreads, 1) void gemm_splitk_kernel(GemmParams p) {
    constexpr int SA = TileOps<256, 128, 4, BPACK, true>::STAGE, SU = TileOps<256, 128, 4, BPACK, false>::STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (SA > SU ? SA : SU)];
    const int tiles = p.tiles_m * p.tiles_n;
    const int L = xcd_logical(blockIdx.x, gridDim.x);
    const int sl = L / tiles;
    if (sl >= p.splits) return;
    int tm, tn;
    grouped_order(L % tiles, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t kbase = (int64_t)sl * p.split_steps * 128;
    if (kbase >= p.K) return;
    const int64_t kbound = min((int64_t)p.split_steps * 128, p.K - kbase);
    const int KS = (int)((kbound + 127) / 128);
    p.c = static_cast<float *>(p.c) + (int64_t)sl * p.c_stride;
    const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 128;
    if ((kbound & 127) == 0)
        gemm_tile<256, 128, 4, BPACK, false, true, 2>(p, m0, p.M, n0, 0, kbase, kbound, KS, smem);
    else
        gemm_tile<256, 128, 4, BPACK, false, false, 2>(p, m0, p.M, n0, 0, kbase, kbound, KS, smem);
}

// C[i] = sum over s of the fp32 partials ws[s * stride + i] in slice order
// (deterministic), i < n; four elements per thread, grid-stride, and the
// last n % 4 one by one.  stride % 4 == 0, ws 16-byte aligned; c 16-byte
// aligned.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ ws, int splits, int64_t n,
                                                            int64_t stride, void *__restrict__ c) {
    const int64_t n4 = n / 4;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < n - n4 * 4) {
        const int64_t i = n4 * 4 + threadIdx.x;
        float a = ws[i];
        for (int sl = 1; sl < splits; ++sl) a += ws[(int64_t)sl * stride + i];
        if constexpr (OUT_BF16) static_cast<uint16_t *>(c)[i] = (uint16_t)f32_to_bf16_rne(a);
        else static_cast<float *>(c)[i] = a;
    }
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        v4f a = reinterpret_cast<const v4f *>(ws)[i];
        for (int sl = 1; sl < splits; ++sl) {
            const v4f b = reinterpret_cast<const v4f *>(ws + (int64_t)sl * stride)[i];
            a = v4f{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
        }
        if constexpr (OUT_BF16) {
            const uint32_t lo = bf16x2_rne(a[0], a[1]);
            const uint32_t hi = bf16x2_rne(a[2], a[3]);
            reinterpret_cast<uint2 *>(c)[i] = uint2{lo, hi};
        } else {
            reinterpret_cast<v4f *>(c)[i] = a;
        }
    }
}

// Dense C in two tile shapes in one launch: workgroups [0, mix_big) take the
// 256x256 tiles of columns [0, 256 * mix_big_cols), the rest the 256x128
// tiles of the remaining columns.  The large tiles come first in dispatch
// order, so they fill the chip's first wave and the small ones the tail.
// Each range is renumbered XCD-aware on its own (mix_big is a multiple of 8,
// so a workgroup's XCD is its id mod 8 in both).
template <bool BPACK, bool OUT_BF16, bool KALIGN, bool SAC = false, bool APACK = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_mixed_kernel(GemmParams p) {
    constexpr int SB = TileOps<256, 256, 2, BPACK, KALIGN, SAC, APACK>::STAGE;
    constexpr int SS = TileOps<256, 128, 4, BPACK, KALIGN, SAC, APACK>::STAGE;
    constexpr int CH = SAC ? 2 * TileOps<256, 256, 2, BPACK, KALIGN, SAC>::CHUNK +
                                 2 * TileOps<256, 256, 2, BPACK, KALIGN, SAC>::CHUNK_B : 0;
    static_assert(2 * (SB > SS ? SB : SS) + CH <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (SB > SS ? SB : SS) + CH];
    const int bid = blockIdx.x;
    int tm, tn;
    if (bid < p.mix_big) {
        grouped_order(xcd_logical(bid, p.mix_big), p.tiles_m, p.mix_big_cols, tm, tn);
        gemm_tile<256, 256, 2, BPACK, OUT_BF16, KALIGN, 2, SAC, false, APACK>(p, (int64_t)tm * 256, p.M,
                                                                              (int64_t)tn * 256, 0, 0, -1, p.KS,
                                                                              smem);
    } else {
        const int n_small = (int)gridDim.x - p.mix_big;
        const int small_cols = n_small / p.tiles_m;
        grouped_order(xcd_logical(bid - p.mix_big, n_small), p.tiles_m, small_cols, tm, tn);
        gemm_tile<256, 128, 4, BPACK, OUT_BF16, KALIGN, 2, SAC, false, APACK>(p, (int64_t)tm * 256, p.M,
                                                                (int64_t)p.mix_big_cols * 256 + (int64_t)tn * 128,
                                                                0, 0, -1, p.KS, smem);
    }
}

// Main loop of one tile for the paired launch below: two-stage ring at LDS
// offsets st_off[0..1] of smem, chunked A scales (K % 512 == 0, packed B) in
// the two chunk buffers at ch_off, chunk c in buffer (c + ch_par) & 1.  Step
// 0's copies and chunk 0 are issued by the caller (into st_off[0] and buffer
// ch_par), which also waits for them and syncs before the call; the loop
// issues and waits for everything after them.
template <int BM, int BN, int WM, bool SAC = true, bool APACK = false>
__device__ __forceinline__ void pair_loop(TileOps<BM, BN, WM, true, true, SAC, APACK> &t, int KS, uint8_t *smem,
                                          const uint32_t *st_off, uint32_t ch_off, int ch_par,
                                          v4f (*acc)[TileOps<BM, BN, WM, true, true, SAC, APACK>::FN]) {
    using T = TileOps<BM, BN, WM, true, true, SAC, APACK>;
    constexpr int FM = T::FM, FN = T::FN;
    int cur = 0;
    for (int ks = 0; ks < KS; ++ks) {
        if (ks) wait_copies_and_sync();    // step ks's copies (step 0: the caller's wait)
        const int c = ks / T::kChunkSteps;
        if constexpr (SAC) {
            if (ks % T::kChunkSteps == 0 && (c + 1) * T::kChunkSteps < KS)
                t.issue_sa_chunk(c + 1, t.lds0 + ch_off + ((c + 1 + ch_par) & 1) * T::CHUNK);
        }
        if (ks + 1 < KS) t.issue2(ks + 1, t.lds0 + st_off[cur ^ 1]);
        const uint8_t *st = smem + st_off[cur];
        int sas[FM], sbs[FN];
        t.lds_scales(st, sas, sbs, smem + ch_off + ((c + ch_par) & 1) * T::CHUNK, ks);
        v8i bf[FN];
        t.lds_bfrags(st, bf);
        t.mma_rows(st, 0, FM, bf, sas, sbs, acc);
        cur ^= 1;
    }
}

// Dense C as pairs of tiles (the mixed tiling with as many 256x128 tiles as
// 256x256 ones, packed B, K % 512 == 0): workgroup i computes the i-th
// 256x256 tile and then the i-th 256x128 tile.  The second tile's first
// copies are issued before the first tile's epilogue, into the LDS the
// first tile no longer reads (its free stage and free scale-chunk buffer);
// the epilogue stages C in the other stage only.  The second tile's loads
// are then in flight while the first tile's C is written, instead of
// starting after it as with one workgroup per tile.
template <bool OUT_BF16, bool APACK = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_pair_kernel(GemmParams p) {
    // chunked A scales, or (APACK) A packed with its per-step scale tiles
    constexpr bool SAC = !APACK;
    using TB = TileOps<256, 256, 2, true, true, SAC, APACK>;
    using TS = TileOps<256, 128, 4, true, true, SAC, APACK>;
    static_assert(TS::STAGE <= TB::STAGE && TS::CHUNK == TB::CHUNK, "small tile inside the large tile's regions");
    constexpr uint32_t SB = TB::STAGE, CH = 2 * TB::STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * TB::STAGE + 2 * TB::CHUNK];
    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int KS = p.KS;
    int tm, tn, tm2, tn2;
    grouped_order(logical, p.tiles_m, p.mix_big_cols, tm, tn);
    const int small_cols = p.tiles_n - p.mix_big_cols;
    grouped_order(logical, p.tiles_m, small_cols, tm2, tn2);
    const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
    const int64_t m2 = (int64_t)tm2 * 256, n2 = (int64_t)p.mix_big_cols * 256 + (int64_t)tn2 * 128;

    // first tile: stages 0 and 1, chunk buffers 0 and 1
    TB tb;
    tb.init(p, m0, p.M, n0, 0, smem);
    v4f acc[TB::FM][TB::FN];
#pragma unroll
    for (int i = 0; i < TB::FM; ++i)
#pragma unroll
        for (int j = 0; j < TB::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (SAC) tb.issue_sa_chunk(0, tb.lds0 + CH);
    tb.issue2(0, tb.lds0);
    wait_copies_and_sync();
    const uint32_t st_b[2] = {0u, SB};
    pair_loop<256, 256, 2, SAC, APACK>(tb, KS, smem, st_b, CH, 0, acc);

    // its last step read stage (KS-1)%2 and chunk buffer ((KS-1)/8)%2; the
    // other stage and buffer are free since the barrier of that step
    const int F = KS & 1, Lc = ((KS - 1) / TB::kChunkSteps) & 1;
    TS ts;
    ts.init(p, m2, p.M, n2, 0, smem);
    if constexpr (SAC) ts.issue_sa_chunk(0, ts.lds0 + CH + (1 - Lc) * TB::CHUNK);
    ts.issue2(0, ts.lds0 + F * SB);

    __syncthreads();                         // every wave is done with the first tile's stages
    {
        const int64_t row0 = m0 + tb.wm * TB::WTM, col0 = n0 + tb.wn * TB::WTN;
        constexpr int ES = OUT_BF16 ? 2 : 4;
        bool counted = false;
        if (n0 + 256 <= p.N && (p.N * ES) % 16 == 0)
            counted = store_tile_lds<TB::FM, TB::FN, OUT_BF16, (int)SB, kWaves, 0>(p, row0, col0, p.M, acc, tb.lane, tb.w,
                                                                        smem + (1 - F) * SB);
        else
            store_tile_scalar<TB::FM, TB::FN, OUT_BF16>(p, row0, col0, p.M, acc, tb.lane);
        // the second tile's first copies have landed; the stores issued after
        // them may still be in flight
        if (counted) __builtin_amdgcn_s_waitcnt(waitcnt_vm(EpilogueShape<TB::FM, TB::FN, OUT_BF16, (int)SB>::kStores));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __syncthreads();                         // the staging area is free again, step 0 visible

    // second tile: step 0 in stage F (issued), step 1 into the other stage
    v4f acc2[TS::FM][TS::FN];
#pragma unroll
    for (int i = 0; i < TS::FM; ++i)
#pragma unroll
        for (int j = 0; j < TS::FN; ++j) acc2[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const uint32_t st_s[2] = {(uint32_t)F * SB, (uint32_t)(1 - F) * SB};
    pair_loop<256, 128, 4, SAC, APACK>(ts, KS, smem, st_s, CH, 1 - Lc, acc2);
    {
        const int64_t row0 = m2 + ts.wm * TS::WTM, col0 = n2 + ts.wn * TS::WTN;
        constexpr int ES = OUT_BF16 ? 2 : 4;
        if (n2 + 128 <= p.N && (p.N * ES) % 16 == 0) {
            __syncthreads();
            store_tile_lds<TS::FM, TS::FN, OUT_BF16, 2 * (int)SB, kWaves, 0>(p, row0, col0, p.M, acc2, ts.lane, ts.w, smem);
        } else {
            store_tile_scalar<TS::FM, TS::FN, OUT_BF16>(p, row0, col0, p.M, acc2, ts.lane);
        }
    }
}

// ------------------------------------------------- copy waves + MFMA waves
// Dense C with both operands packed (K % 128 == 0) as a persistent launch of
// 256x128 tiles whose waves split the work: waves 0-3 (one per SIMD) only
// compute, each a 128x64 block of the tile; waves 4-7 (the other wave of
// each SIMD) only copy, each a quarter of every k-step's A and B tiles and
// scale tiles.  Measured in the two-stage kernels above: the wave that issues
// a step's copies is held in the issue for most of the step while the memory
// pipeline drains, and a step's copies land ~1000 clocks after the last one
// is issued, so copy issue plus the issuing wave's own MFMAs set the step.
// Here no computing wave ever issues a copy, and three 49.5 KB stages form a
// ring that runs on across tile boundaries, so two steps of copies are in
// flight while one is computed (a 256x256 tile's three stages would not fit
// the LDS).  One barrier per step g: before it, the computing waves have
// finished step g and the copying waves have seen step g+1's copies land;
// after it, step g+1 is computed and the copies of step g+3 go into the stage
// step g used.  C leaves from the accumulators through a descriptor spanning
// this wave's block of C (bf16: 16-row bands through a 2.3 KB LDS buffer per
// wave, so every store writes whole 128-byte rows; fp32: 16 bytes per lane
// and 16x16 tile); the stores drain while the next tile's steps run, since
// the computing waves never wait on vector memory.
struct WsLayout {
    static constexpr int BM = 256, BN = 128, NST = 3;
    static constexpr int A_OFF = 0, B_OFF = BM * 128;            // 32 KB of A rows, 16 KB of B rows
    static constexpr int SA_OFF = B_OFF + BN * 128;              // the A panel's 1 KB scale tile
    static constexpr int SB_OFF = SA_OFF + BM * 4;               // 512 B: the B half panel's 8 atoms
    static constexpr int STAGE = SB_OFF + BN * 4;
    static constexpr int FM = 8, FN = 4;                         // 128x64 per computing wave
    // bf16 C leaves each computing wave 16 rows at a time through a band
    // buffer of its own after the ring (rows padded by 16 bytes)
    static constexpr int BAND_ROW = 64 * 2 + 16, BAND = 16 * BAND_ROW, BAND_OFF = NST * STAGE;
    // grouped launch: the coordinates of a workgroup's tiles (at most UNITS),
    // found once before the first copy
    static constexpr int UNITS = 64, UNIT_OFF = BAND_OFF + 4 * BAND;
};
static_assert(WsLayout::UNIT_OFF + WsLayout::UNITS * 16 <= 160 * 1024, "ring, band buffers and tile table fit the LDS");

// a grouped tile: expert, first and end rows (of the padded row space), tile column
struct WsUnit {
    int g, m0, m_end, tn;
};

// copy instructions one copying wave (0..3) issues per k-step
__device__ __forceinline__ constexpr int ws_copies(int pw) { return 8 + 4 + 1 + (pw < 2 ? 1 : 0); }

// the tiles of workgroup `wg`: each XCD (wg % 8) owns a contiguous share of
// the tile order in proportion to its workgroups, dealt over them; returns
// the first tile, the stride and the count
__device__ __forceinline__ void ws_tiles(int wg, int nwg, int T, int &first, int &stride, int &count) {
    const int q = nwg / 8, r = nwg % 8, x = wg % 8, j = wg / 8;
    const int nx = q + (x < r ? 1 : 0);
    const int before = x * q + (x < r ? x : r);                  // workgroups on XCDs < x
    const int lo = (int)((int64_t)T * before / nwg), hi = (int)((int64_t)T * (before + nx) / nwg);
    first = lo + j;
    stride = nx;
    count = first < hi ? (hi - first + nx - 1) / nx : 0;
}

template <bool OUT_BF16, bool GROUPED = false, bool GK = false, bool HALF = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_ws_kernel(GemmParams p) {
    static_assert(!(GROUPED && GK), "grouped rows or grouped K");
    // HALF (dense): 128-row tiles (p.tiles_m counts them), the upper or lower
    // half of a 256-row panel; only the computing waves of rows 0..127 work
    // and only those rows' A bytes and scales are copied
    static_assert(!HALF || (!GROUPED && !GK), "half tiles are dense");
    using Lw = WsLayout;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[Lw::UNIT_OFF + (GROUPED ? Lw::UNITS * 16 : 0)];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = p.KS;
    // work units: tile u % T over K slice u / T (p.splits > 1: the split
    // launch, fp32 partials of slice s at c + s * c_stride; else one slice).
    // Grouped: the m-tiles are each expert's 256-row tiles in expert order
    // (clamped offsets, as find_group), the packed A rows those of the
    // padded row space, the launch never split.  GK (the experts' weight
    // gradients): tile u % T of expert u / T over the expert's k-steps
    // [offsets[g] / 128, offsets[g+1] / 128) of the packed token axis (ranges
    // clamped into [0, K]), its C at c + g * c_stride
    const int tiles_m =
        GROUPED ? __builtin_amdgcn_readfirstlane(count_group_tiles<256>(p.offsets, p.G, p.M, lane)) : p.tiles_m;
    const int T = tiles_m * p.tiles_n;
    const int S = GK ? p.G : (p.splits > 1 ? p.splits : 1), L = p.splits > 1 ? p.split_steps : KS;
    int first, stride, nunit;
    if constexpr (GK) {
        // the experts' tiles in dispatch order, every workgroup taking units
        // blockIdx, blockIdx + grid, ...: an expert's 1 to ~60 k-steps per
        // tile vary too much for contiguous per-XCD shares of the units, and
        // consecutive units (one expert's tiles) land on different workgroups
        first = blockIdx.x;
        stride = gridDim.x;
        nunit = first < T * S ? (T * S - first + stride - 1) / stride : 0;
    } else {
        ws_tiles(blockIdx.x, gridDim.x, T * S, first, stride, nunit);
    }
    // GK: an expert without tokens runs one step whose copies all read out of
    // range (zeros), so its C is stored as zeros by the common epilogue
    auto gk_empty = [&](int i) -> bool {
        if constexpr (GK) {
            const int g = (first + i * stride) / T;
            int64_t lo = p.offsets[g], hi = p.offsets[g + 1];
            lo = lo < 0 ? 0 : (lo > p.K ? p.K : lo);
            hi = hi < lo ? lo : (hi > p.K ? p.K : hi);
            return __builtin_amdgcn_readfirstlane((int)(hi > lo)) == 0;
        } else {
            return false;
        }
    };
    auto unit_steps = [&](int i, int &k0, int &k1) {
        if constexpr (GK) {
            const int g = (first + i * stride) / T;
            int64_t lo = p.offsets[g], hi = p.offsets[g + 1];
            lo = lo < 0 ? 0 : (lo > p.K ? p.K : lo);
            hi = hi < lo ? lo : (hi > p.K ? p.K : hi);
            k0 = __builtin_amdgcn_readfirstlane((int)(lo / 128));
            k1 = __builtin_amdgcn_readfirstlane((int)((hi + 127) / 128));
            if (k1 == k0) k1 = k0 + 1;
        } else {
            k0 = (first + i * stride) / T * L;
            k1 = min(KS, k0 + L);
        }
    };
    WsUnit *units = reinterpret_cast<WsUnit *>(smem + Lw::UNIT_OFF);
    if constexpr (GROUPED) {
        // the launcher keeps every workgroup's tile count within UNITS
        nunit = min(nunit, Lw::UNITS);
        for (int i = w; i < nunit; i += kWaves) {
            int tm, tn;
            grouped_order((first + i * stride) % T, tiles_m, p.tiles_n, tm, tn);
            int64_t glo = 0, ghi = 0;
            int tig = 0;
            const int g = find_group<256>(p.offsets, p.G, p.M, tm, lane, glo, ghi, tig);
            const int64_t m0 = glo + (int64_t)tig * 256;
            if (lane == 0) units[i] = g < 0 ? WsUnit{0, 0, 0, tn} : WsUnit{g, (int)m0, (int)ghi, tn};
        }
        __syncthreads();
    }
    int total = 0;                                               // k-steps of this workgroup
    for (int i = 0; i < nunit; ++i) {
        int k0, k1;
        unit_steps(i, k0, k1);
        total += k1 - k0;
    }
    const uint32_t lds0 = lds_addr(smem);

    if (w >= 4) {
        // ---- copying wave pw: segments pw, pw + 4, ... of each step
        const int pw = w - 4;
        const int nc = ws_copies(pw) - (HALF ? 4 : 0);
        int iu = 0, ks = 0, kend = 0, st = 0;                    // next step to issue
        v4i ra = {}, rsa = {}, rb = {}, rsb = {};
        int a_m0 = 0, a_rows = 0;                                // grouped: the tile's rows in A's first panel
        uint32_t zero_oob = 0;                                   // GK: kOOB for an expert without tokens
        auto set_tile = [&](int i) {
            zero_oob = gk_empty(i) ? kOOB : 0u;
            int tm, tn;
            int64_t pa, bp = 0;
            if constexpr (GROUPED) {
                const WsUnit u = units[i];
                const int g = __builtin_amdgcn_readfirstlane(u.g), m0 = __builtin_amdgcn_readfirstlane(u.m0);
                a_rows = min(__builtin_amdgcn_readfirstlane(u.m_end) - m0, Lw::BM);
                tn = __builtin_amdgcn_readfirstlane(u.tn);
                pa = m0 / kPanelRows;
                a_m0 = m0 % kPanelRows;
                bp = (int64_t)g * p.NP;
            } else {
                grouped_order((first + i * stride) % T, p.tiles_m, p.tiles_n, tm, tn);
                pa = HALF ? tm / 2 : tm;
                a_m0 = HALF ? (tm % 2) * 128 : 0;
            }
            // A: one panel, or (grouped, a tile starting inside a panel) two
            const int64_t na = GROUPED ? min((int64_t)2, (p.M + kPanelRows - 1) / kPanelRows - pa) : 1;
            const int64_t pb = bp + ((int64_t)tn * Lw::BN) / kPanelRows, prow = ((int64_t)tn * Lw::BN) % kPanelRows;
            ra = make_srd(p.a_q + pa * KS * kTileBytes, (uint32_t)(na * KS * kTileBytes));
            rsa = make_srd(p.a_s + pa * KS * kScaleStepBytes, (uint32_t)(na * KS * kScaleStepBytes));
            rb = make_srd(p.b_q + pb * KS * kTileBytes + prow * 128,
                          (uint32_t)((int64_t)KS * kTileBytes - prow * 128));
            rsb = make_srd(p.b_s + pb * KS * kScaleStepBytes + (prow / 16) * 64,
                           (uint32_t)((int64_t)KS * kScaleStepBytes - (prow / 16) * 64));
        };
        // the first unit from i on that has steps (GK: past empty experts)
        auto start_unit = [&](int i) {
            for (iu = i; iu < nunit; ++iu) {
                unit_steps(iu, ks, kend);
                if (ks < kend) break;
            }
            if (iu < nunit) set_tile(iu);
        };
        start_unit(0);
        auto issue_next = [&]() {
            const uint32_t sbase = lds0 + st * Lw::STAGE;
            const uint32_t k0 = (uint32_t)ks * (uint32_t)kTileBytes;
#pragma unroll
            for (int i = 0; i < (HALF ? 4 : 8); ++i) {
                const int seg = i * 4 + pw;
                uint32_t off = k0 + (HALF ? (uint32_t)a_m0 * 128u : 0u) + seg * 1024 + lane * 16;
                if constexpr (GROUPED) {
                    // the tile's rows seg*8 .. +7, in the panel they lie in;
                    // rows past the expert's read zeros
                    const int r = a_m0 + seg * 8;
                    off = seg * 8 < a_rows ? (uint32_t)(r / kPanelRows) * (uint32_t)KS * (uint32_t)kTileBytes + k0 +
                                                 (uint32_t)(r % kPanelRows) * 128u + lane * 16
                                           : kOOB;
                }
                dma16(ra, off | zero_oob, sbase + Lw::A_OFF + seg * 1024);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int seg = i * 4 + pw;
                dma16(rb, (k0 + seg * 1024 + lane * 16) | zero_oob, sbase + Lw::B_OFF + seg * 1024);
            }
            const uint32_t s0 = (uint32_t)ks * (uint32_t)kScaleStepBytes + pw * 256 + lane * 4;
            uint32_t sa_off = s0;
            if constexpr (GROUPED) {
                // this lane's dword: atom pw*4 + lane/16 of the tile (16 rows)
                const int ra16 = (pw * 4 + (lane >> 4)) * 16, r = a_m0 + ra16;
                sa_off = ra16 < a_rows ? (uint32_t)(r / kPanelRows) * (uint32_t)KS * (uint32_t)kScaleStepBytes +
                                             (uint32_t)ks * (uint32_t)kScaleStepBytes +
                                             (uint32_t)((r % kPanelRows) >> 4) * 64u + (lane & 15) * 4
                                       : kOOB;
            }
            if constexpr (HALF) sa_off = pw < 2 ? s0 + (uint32_t)a_m0 * 4u : kOOB;   // the half's 8 atoms
            dma4(rsa, sa_off | zero_oob, sbase + Lw::SA_OFF + pw * 256);
            if (pw < 2) dma4(rsb, s0 | zero_oob, sbase + Lw::SB_OFF + pw * 256);
            st = st == Lw::NST - 1 ? 0 : st + 1;
            if (++ks == kend) start_unit(iu + 1);
        };
        auto wait_all_but_last = [&]() {
            if constexpr (HALF) {
                if (nc == 10) __builtin_amdgcn_s_waitcnt(waitcnt_vm(10));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
            } else {
                if (nc == 14) __builtin_amdgcn_s_waitcnt(waitcnt_vm(14));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(13));
            }
        };
        if (total > 0) issue_next();
        if (total > 1) { issue_next(); wait_all_but_last(); }
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();                                         // step 0 has landed
        for (int g = 0; g < total; ++g) {
            if (g + 2 < total) {
                issue_next();                                    // into the stage step g - 1 used
                wait_all_but_last();                             // step g + 1 has landed
            } else {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            }
            __syncthreads();
        }
        return;
    }

    // ---- computing wave: rows wm * 128.., columns wn * 64.. of the tile
    const int wm = w >> 1, wn = w & 1;
    constexpr int FM = Lw::FM, FN = Lw::FN;
    constexpr int ES = OUT_BF16 ? 2 : 4;
    const int g16 = lane >> 4;                                   // lane group: columns 4 g16 .. 4 g16 + 3
    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // the unit's C (or its slice's fp32 partial) from the accumulators, which
    // are then cleared
    auto store_unit = [&](int iu) {
        // this wave's rows and columns that lie inside C
        const int u = first + iu * stride;
        int tm, tn;
        int64_t row0, row_end;
        if constexpr (GROUPED) {
            const WsUnit un = units[iu];
            tn = __builtin_amdgcn_readfirstlane(un.tn);
            row0 = (int64_t)__builtin_amdgcn_readfirstlane(un.m0) + wm * 128;
            row_end = __builtin_amdgcn_readfirstlane(un.m_end);
        } else if constexpr (HALF) {
            // rows tm*128 .. +127 (the wm = 1 waves hold none)
            grouped_order(u % T, p.tiles_m, p.tiles_n, tm, tn);
            row0 = (int64_t)tm * 128 + wm * 128;
            row_end = min(p.M, (int64_t)tm * 128 + 128);
        } else {
            grouped_order(u % T, p.tiles_m, p.tiles_n, tm, tn);
            row0 = (int64_t)tm * Lw::BM + wm * 128;
            row_end = p.M;
        }
        const int64_t col0 = (int64_t)tn * Lw::BN + wn * 64;
        const int64_t rows_here = row_end - row0, cols_here = p.N - col0;
        uint8_t *cbase = static_cast<uint8_t *>(p.c) + (S > 1 ? (int64_t)(u / T) * p.c_stride * ES : 0);
        if (rows_here > 0 && cols_here > 0) {
            const int rh = (int)min(rows_here, (int64_t)128), chh = (int)min(cols_here, (int64_t)64);
            const uint32_t range = (uint32_t)(((int64_t)(rh - 1) * p.N + chh) * ES);
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(cbase + (row0 * p.N + col0) * ES, range);
            const int r0 = lane & 15;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = i * 16 + r0;
                if constexpr (OUT_BF16) {
                    // the band of 16 rows through this wave's LDS band
                    // buffer, out as 8 whole 128-byte rows per store
                    uint8_t *band = smem + Lw::BAND_OFF + w * Lw::BAND;
#pragma unroll
                    for (int jj = 0; jj < FN; ++jj)
                        *reinterpret_cast<v2i *>(band + r0 * Lw::BAND_ROW + jj * 32 + g16 * 8) =
                            v2i{(int)bf16x2_rne(acc[i][jj][0], acc[i][jj][1]),
                                (int)bf16x2_rne(acc[i][jj][2], acc[i][jj][3])};
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int rr = h * 8 + (lane >> 3), cl = (lane & 7) * 8, row = i * 16 + rr;
                        const v4i v = *reinterpret_cast<const v4i *>(band + rr * Lw::BAND_ROW + (lane & 7) * 16);
                        const uint32_t off =
                            (row < rh && cl < chh) ? (uint32_t)(((int64_t)row * p.N + cl) * ES) : kOOB;
                        __builtin_amdgcn_raw_buffer_store_b128(v, rc, (int)off, 0, kStoreStream);
                    }
                    __builtin_amdgcn_wave_barrier();
                } else {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int cl = j * 16 + g16 * 4;
                        const uint32_t off = (r < rh && cl < chh) ? (uint32_t)(((int64_t)r * p.N + cl) * ES) : kOOB;
                        // (GK: the experts' gradients are written once, streamed)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            v4i{(int)float_to_bits(acc[i][j][0]), (int)float_to_bits(acc[i][j][1]),
                                (int)float_to_bits(acc[i][j][2]), (int)float_to_bits(acc[i][j][3])},
                            rc, (int)off, 0, GK ? kStoreStream : 0);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    };
    __syncthreads();                                             // step 0 has landed
    int st = 0;
    for (int iu = 0; iu < nunit; ++iu) {
        int k0, k1;
        unit_steps(iu, k0, k1);
        for (int ks = k0; ks < k1; ++ks) {
            const uint8_t *sp = smem + st * Lw::STAGE;
            const uint8_t *sa = sp + Lw::A_OFF + wm * 128 * 128;
            if (!HALF || wm == 0) {
                int sas[FM], sbs[FN];
                v8i bf[FN], af[2];
                // the B fragments and scales, then row 0's A fragment; each later
                // A fragment is read while the previous row's MFMAs run (with one
                // computing wave per SIMD nothing else hides the LDS latency)
#pragma unroll
                for (int j = 0; j < FN; ++j) bf[j] = lds_frag(sp + Lw::B_OFF + (wn * 64 + j * 16) * 128, lane);
#pragma unroll
                for (int j = 0; j < FN; ++j) sbs[j] = sp[Lw::SB_OFF + (wn * FN + j) * 64 + lane];
#pragma unroll
                for (int i = 0; i < FM; ++i) sas[i] = sp[Lw::SA_OFF + (wm * FM + i) * 64 + lane];
                af[0] = lds_frag(sa, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    if (i + 1 < FM) af[(i + 1) & 1] = lds_frag(sa + (i + 1) * 16 * 128, lane);
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i & 1], acc[i][j], 0, 0,
                                                                                     0, sbs[j], 0, sas[i]);
                    __builtin_amdgcn_sched_barrier(0);      // keep the read of row i + 1 ahead of row i's MFMAs
                }
            }
            st = st == Lw::NST - 1 ? 0 : st + 1;
            if (ks == k1 - 1) store_unit(iu);
            __syncthreads();
        }
    }
}

// Grouped (MoE) GEMM with 256x256 tiles as a persistent launch: one
// workgroup per CU walks tiles; each XCD (workgroup id mod 8) takes a
// contiguous eighth of the tiles that exist, dealt over its workgroups.
// Between two tiles the next tile's first copies (and scale chunk) go into
// the stage and chunk buffer the finished tile's last step did not read,
// before its epilogue, which stages C in the other stage only -- the same
// hand-over as gemm_pair_kernel.  Packed B, K % 128 == 0; SAC: K % 512 == 0;
// APACK: A in the packed layout too (the copies of each 8-row segment are one
// contiguous KB wherever the group's tile starts).
template <bool OUT_BF16, bool SAC, bool APACK = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_grouped_persist_kernel(GemmParams p) {
    static_assert(!(SAC && APACK), "packed A carries its scales per step");
    using T = TileOps<256, 256, 2, true, true, SAC, APACK>;
    constexpr uint32_t SB = T::STAGE, CH = 2 * T::STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::STAGE + (SAC ? 2 * T::CHUNK : 0)];
    const int lane = threadIdx.x & 63;
    const int tiles_m = count_group_tiles<256>(p.offsets, p.G, p.M, lane);
    const int n = tiles_m * p.tiles_n;
    // this workgroup's tiles: XCD x = blockIdx % 8 owns [lo_x, hi_x), its
    // workgroups (blockIdx / 8 = j of nj) take lo_x + j, lo_x + j + nj, ...
    const int G8 = (int)gridDim.x;
    const int x = blockIdx.x % 8, j = blockIdx.x / 8, nj = (G8 - x + 7) / 8;
    const int lo = (int)((int64_t)n * x / 8), hi = (int)((int64_t)n * (x + 1) / 8);
    int L = lo + j;
    if (L >= hi) return;
    const int KS = p.KS;

    auto coords = [&](int Lt, int64_t &m0, int64_t &m_end, int64_t &n0, int64_t &g) -> bool {
        int tm, tn;
        grouped_order(Lt, tiles_m, p.tiles_n, tm, tn);
        int64_t glo, ghi;
        int tig;
        const int gg = find_group<256>(p.offsets, p.G, p.M, tm, lane, glo, ghi, tig);
        if (gg < 0) return false;
        g = gg;
        m0 = glo + (int64_t)tig * 256;
        m_end = ghi;
        n0 = (int64_t)tn * 256;
        return true;
    };
    int64_t m0, m_end, n0, g;
    if (!coords(L, m0, m_end, n0, g)) return;
    T t;
    t.init(p, m0, m_end, n0, g, smem);
    if constexpr (SAC) t.issue_sa_chunk(0, t.lds0 + CH);
    t.issue2(0, t.lds0);
    wait_copies_and_sync();
    uint32_t st[2] = {0u, SB};
    int ch_par = 0;
    while (true) {
        v4f acc[T::FM][T::FN];
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < T::FN; ++jj) acc[i][jj] = v4f{0.f, 0.f, 0.f, 0.f};
        pair_loop<256, 256, 2, SAC, APACK>(t, KS, smem, st, CH, ch_par, acc);
        // the last step read st[(KS-1)&1] and chunk buffer
        // ((KS-1)/8 + ch_par)&1; the other stage and buffer are free
        const uint32_t st_free = st[KS & 1], st_busy = st[(KS - 1) & 1];
        const int c_free = 1 - ((((KS - 1) / T::kChunkSteps) + ch_par) & 1);
        const int64_t row0 = m0 + t.wm * T::WTM, col0 = n0 + t.wn * T::WTN, mend = m_end;
        const int wm = t.wm;
        (void)wm;
        L += nj;
        int64_t nm0 = 0, nm_end = 0, nn0 = 0, ng = 0;
        // uniform over the workgroup (the coordinates come from wave-wide
        // scans), said so the descriptors stay scalar through the loop
        const bool more = __builtin_amdgcn_readfirstlane((int)(L < hi && coords(L, nm0, nm_end, nn0, ng))) != 0;
        T t2;
        if (more) {
            t2.init(p, nm0, nm_end, nn0, ng, smem);
            if constexpr (SAC) t2.issue_sa_chunk(0, t2.lds0 + CH + c_free * T::CHUNK);
            t2.issue2(0, t2.lds0 + st_free);
        }
        __syncthreads();                     // every wave is done with the finished tile's stages
        bool counted = false;
        {
            constexpr int ES = OUT_BF16 ? 2 : 4;
            if (n0 + 256 <= p.N && (p.N * ES) % 16 == 0)
                counted = store_tile_lds<T::FM, T::FN, OUT_BF16, (int)SB>(p, row0, col0, mend, acc, t.lane,
                                                                         t.w, smem + st_busy);
            else
                store_tile_scalar<T::FM, T::FN, OUT_BF16>(p, row0, col0, mend, acc, t.lane);
        }
        if (!more) break;
        // the next tile's first copies have landed; the finished tile's
        // stores, issued after them, drain behind the next tile's steps
        if (counted) __builtin_amdgcn_s_waitcnt(waitcnt_vm(EpilogueShape<T::FM, T::FN, OUT_BF16, (int)SB>::kStores));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();                     // the staging stage is free again, step 0 visible
        t = t2;
        m0 = nm0; m_end = nm_end; n0 = nn0; g = ng;
        st[0] = st_free;
        st[1] = st_busy;
        ch_par = c_free;
    }
}

// Pipeline depth.  Measured: a third stage (where it fits the LDS) speeds up
// the grouped expert GEMMs (short K per tile: 443 -> 412 us and 315 -> 301 us
// on the MoE layer) but slows the dense 256x128 qkv GEMM (127 -> 136 us), so
// only grouped launches take it.
template <int BM, int BN, int WM, bool BP, bool GROUPED>
constexpr int kStages3 = GROUPED && 3 * TileOps<BM, BN, WM, BP, true>::STAGE <= 160 * 1024 ? 3 : 2;

// Dense launches with K % 512 == 0 (A scale rows a multiple of 16 bytes, so
// every 16-byte piece of a chunk lies wholly inside or wholly past its row)
// copy the A scales in chunks of 8 k-steps instead of a dword per row per
// step.  Each per-step copy touches one 128-byte line per row, as many line
// requests as the step's whole A tile; measured on MI355X the chunked copy
// takes 8192x24576x4096 from 782 to 743 us, 8192x4096x12288 from 362 to
// 347 us and the canonical-B 24576x4096x8192 from 775 to 749 us.
static bool chunked_a_scales(int64_t K) { return K % 512 == 0; }

template <int BM, int BN, int WM, bool GROUPED>
static hipError_t launch_tile(const GemmParams &p, bool b_packed, bool c_bf16, int nwg, hipStream_t s) {
    dim3 grid((unsigned)nwg), block(kThreads);
    const bool kal = p.K % 128 == 0;
    // (dense tiles, and grouped 256-row tiles, which keep the two-stage ring)
    if constexpr (!GROUPED || (BM == 256 && kStages3<BM, BN, WM, true, GROUPED> == 2 &&
                               kStages3<BM, BN, WM, false, GROUPED> == 2)) {
        if (chunked_a_scales(p.K)) {
#define MX_LAUNCHC(BP, BF) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, BP, BF, GROUPED, true, false, 2, true>), grid, block, 0, s, p)
            if (b_packed) { if (c_bf16) MX_LAUNCHC(true, true); else MX_LAUNCHC(true, false); }
            else { if (c_bf16) MX_LAUNCHC(false, true); else MX_LAUNCHC(false, false); }
#undef MX_LAUNCHC
            return hipGetLastError();
        }
    }
#define MX_LAUNCH2(BP, BF, KA) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, BP, BF, GROUPED, KA>), grid, block, 0, s, p)
#define MX_LAUNCH3(BP, BF) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, BP, BF, GROUPED, true, false, kStages3<BM, BN, WM, BP, GROUPED>>), grid, block, 0, s, p)
    if (kal) {
        if (b_packed) { if (c_bf16) MX_LAUNCH3(true, true); else MX_LAUNCH3(true, false); }
        else { if (c_bf16) MX_LAUNCH3(false, true); else MX_LAUNCH3(false, false); }
    } else {
        if (b_packed) { if (c_bf16) MX_LAUNCH2(true, true, false); else MX_LAUNCH2(true, false, false); }
        else { if (c_bf16) MX_LAUNCH2(false, true, false); else MX_LAUNCH2(false, false, false); }
    }
#undef MX_LAUNCH2
#undef MX_LAUNCH3
    return hipGetLastError();
}

// Dense tile shapes.  A 256x256 tile moves 1.0 byte of operands per output
// per k-step, a 256x128 tile 1.5, and the copy path from L2 into LDS is the
// kernels' limit: measured per k-step, a 256x128 tile takes ~0.66 of a
// 256x256 tile's time.  With one workgroup per CU, the launch takes as many
// rounds of tiles as ceil(tiles / CUs); the choice minimises the estimated
// total: all 256x256, all 256x128, or whole rounds of 256x256 tiles over
// the leading columns followed by 256x128 tiles over the rest.
DenseTiling dense_tiling(int64_t M, int64_t N, int cus) {
    constexpr double kSmall = 0.66;
    const int64_t tm = ceil_div(M, 256), tn_big = ceil_div(N, 256), tn_small = ceil_div(N, 128);
    DenseTiling best{(int)tn_big, 0};
    double best_t = (double)ceil_div(tm * tn_big, (int64_t)cus);
    if (N <= 128) return best;
    const double t_small = kSmall * (double)ceil_div(tm * tn_small, (int64_t)cus);
    if (t_small < best_t) {
        best = DenseTiling{0, (int)tn_small};
        best_t = t_small;
    }
    // whole rounds of large tiles, whole tile columns, workgroup count a multiple of 8
    for (int64_t rounds = 1; rounds * cus < tm * tn_big; ++rounds) {
        int64_t cols = rounds * cus / tm;
        while (cols > 0 && (tm * cols) % 8 != 0) --cols;
        if (cols <= 0 || cols >= tn_big) continue;
        const int64_t rest = ceil_div(N - cols * 256, 128);
        const double t = (double)ceil_div(tm * cols, (int64_t)cus) + kSmall * (double)ceil_div(tm * rest, (int64_t)cus);
        if (t < best_t - 1e-9) {
            best = DenseTiling{(int)cols, (int)rest};
            best_t = t;
        }
    }
    return best;
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
    p.lda = K; p.lsa = K / 32; p.ldb = K; p.lsb = K / 32;
    const int cus = device_cu_count();
    const DenseTiling d = dense_tiling(M, N, cus);
    p.tiles_m = (int)ceil_div(M, 256);
    if (d.big_cols > 0 && d.small_cols > 0) {
        p.tiles_n = d.big_cols + d.small_cols;
        p.mix_big = p.tiles_m * d.big_cols;
        p.mix_big_cols = d.big_cols;
        dim3 grid((unsigned)(p.mix_big + p.tiles_m * d.small_cols)), block(kThreads);
        const bool kal = K % 128 == 0;
#define MX_MIXED(BP, BF, KA) hipLaunchKernelGGL((gemm_mixed_kernel<BP, BF, KA>), grid, block, 0, stream, p)
#define MX_MIXEDC(BP, BF) hipLaunchKernelGGL((gemm_mixed_kernel<BP, BF, true, true>), grid, block, 0, stream, p)
        if (b_packed && chunked_a_scales(K) && d.small_cols == d.big_cols) {
            // as many 256x128 tiles as 256x256 ones: one workgroup per pair
            // (measured on the qkv layer, 4096x6144x4096: 1.5-3% faster than
            // one workgroup per tile, bit-identical)
            dim3 pgrid((unsigned)p.mix_big);
            if (c_bf16) hipLaunchKernelGGL((gemm_pair_kernel<true>), pgrid, block, 0, stream, p);
            else hipLaunchKernelGGL((gemm_pair_kernel<false>), pgrid, block, 0, stream, p);
        } else if (chunked_a_scales(K)) {
            if (b_packed) { if (c_bf16) MX_MIXEDC(true, true); else MX_MIXEDC(true, false); }
            else { if (c_bf16) MX_MIXEDC(false, true); else MX_MIXEDC(false, false); }
        } else if (kal) {
            if (b_packed) { if (c_bf16) MX_MIXED(true, true, true); else MX_MIXED(true, false, true); }
            else { if (c_bf16) MX_MIXED(false, true, true); else MX_MIXED(false, false, true); }
        } else {
            if (b_packed) { if (c_bf16) MX_MIXED(true, true, false); else MX_MIXED(true, false, false); }
            else { if (c_bf16) MX_MIXED(false, true, false); else MX_MIXED(false, false, false); }
        }
#undef MX_MIXED
#undef MX_MIXEDC
        return hipGetLastError();
    }
    if (d.big_cols > 0) {
        p.tiles_n = d.big_cols;
        return launch_tile<256, 256, 2, false>(p, b_packed, c_bf16, p.tiles_m * p.tiles_n, stream);
    }
    p.tiles_n = d.small_cols;
    return launch_tile<256, 128, 4, false>(p, b_packed, c_bf16, p.tiles_m * p.tiles_n, stream);
}

// The tiles of launch_gemm_packed.  Where gemm_ws_kernel's 256x128 tiles
// make at most three rounds over the CUs (its persistent walk hides each
// tile's prologue) the choice weighs each candidate's rounds by the time of
// one of its k-steps, which the copies into LDS set: 1 for 256x128 tiles,
// ~0.67 for 128x128 ones (two thirds of the bytes), ~1.5 for the two-stage
// 256x256 tiles (measured 1850-2050 against ~3100 clocks per step).  Beyond
// three rounds, or where the epilogue's stores cannot take the walk (N not a
// multiple of 16 bytes of C, or 128 rows of C past 2 GB), launch_gemm's tilings.
PackedTiling packed_tiling(int64_t M, int64_t N, bool c_bf16, int cus) {
    const int64_t tm = ceil_div(M, 256), full = tm * ceil_div(N, 128);
    if (N % (c_bf16 ? 8 : 4) != 0 || (int64_t)128 * N * (c_bf16 ? 2 : 4) >= ((int64_t)1 << 31) ||
        full > (int64_t)3 * cus)
        return PackedTiling::kDense;
    const double t_full = (double)ceil_div(full, (int64_t)cus);
    const double t_half = 0.67 * (double)ceil_div(ceil_div(M, 128) * ceil_div(N, 128), (int64_t)cus);
    const double t_big = 1.5 * (double)ceil_div(tm * ceil_div(N, 256), (int64_t)cus);
    if (t_big < t_full - 1e-9 && t_big < t_half - 1e-9) return PackedTiling::kDense;
    return t_half < t_full - 1e-9 ? PackedTiling::kWsHalf : PackedTiling::kWs;
}

// Both operands in the packed layout (A quantized straight into it, or
// repacked): every copy of a k-step reads one contiguous 1 KB, where a
// canonical A segment gathers 8 rows K bytes apart.  K % 128 == 0.  The
// tiles of packed_tiling.
hipError_t launch_gemm_packed(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q, const uint8_t *b_s,
                              int64_t M, int64_t N, int64_t K, void *c, bool c_bf16, hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = c;
    p.M = M; p.N = N; p.K = K;
    p.KS = (int)packed_ksteps(K);
    p.NP = (int)packed_panels(N);
    p.G = 1;
    p.offsets = nullptr;
    p.lda = K; p.lsa = K / 32; p.ldb = K; p.lsb = K / 32;
    const int cus = device_cu_count();
    p.tiles_m = (int)ceil_div(M, 256);
    dim3 block(kThreads);
    const PackedTiling pt = packed_tiling(M, N, c_bf16, cus);
    if (pt == PackedTiling::kWs || pt == PackedTiling::kWsHalf) {
        const bool half = pt == PackedTiling::kWsHalf;
        if (half) p.tiles_m = (int)ceil_div(M, 128);
        p.tiles_n = (int)ceil_div(N, 128);
        dim3 grid((unsigned)std::min<int64_t>((int64_t)p.tiles_m * p.tiles_n, cus));
        if (half) {
            if (c_bf16) hipLaunchKernelGGL((gemm_ws_kernel<true, false, false, true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((gemm_ws_kernel<false, false, false, true>), grid, block, 0, stream, p);
        } else {
            if (c_bf16) hipLaunchKernelGGL((gemm_ws_kernel<true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((gemm_ws_kernel<false>), grid, block, 0, stream, p);
        }
        return hipGetLastError();
    }
    const DenseTiling d = dense_tiling(M, N, cus);
    if (d.big_cols > 0 && d.small_cols > 0) {
        p.tiles_n = d.big_cols + d.small_cols;
        p.mix_big = p.tiles_m * d.big_cols;
        p.mix_big_cols = d.big_cols;
        if (d.small_cols == d.big_cols) {
            dim3 grid((unsigned)p.mix_big);
            if (c_bf16) hipLaunchKernelGGL((gemm_pair_kernel<true, true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((gemm_pair_kernel<false, true>), grid, block, 0, stream, p);
        } else {
            dim3 grid((unsigned)(p.mix_big + p.tiles_m * d.small_cols));
            if (c_bf16) hipLaunchKernelGGL((gemm_mixed_kernel<true, true, true, false, true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((gemm_mixed_kernel<true, false, true, false, true>), grid, block, 0, stream, p);
        }
        return hipGetLastError();
    }
    if (d.big_cols > 0) {
        p.tiles_n = d.big_cols;
        dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
        if (c_bf16)
            hipLaunchKernelGGL((gemm_kernel<256, 256, 2, true, true, false, true, false, 2, false, false, true>), grid,
                               block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<256, 256, 2, true, false, false, true, false, 2, false, false, true>), grid,
                               block, 0, stream, p);
        return hipGetLastError();
    }
    p.tiles_n = d.small_cols;
    dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    if (c_bf16)
        hipLaunchKernelGGL((gemm_kernel<256, 128, 4, true, true, false, true, false, 2, false, false, true>), grid,
                           block, 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<256, 128, 4, true, false, false, true, false, 2, false, false, true>), grid,
                           block, 0, stream, p);
    return hipGetLastError();
}

// Packed A and B with K split into slices (the plan of splitk_plan): the
// copying / computing-wave launch walks (tile, slice) units and writes each
// slice's fp32 partial tile to `workspace` + slice * c_stride (the layout of
// gemm_splitk_kernel's partials), then splitk_reduce_kernel sums them in
// slice order.  Each partial is the same MFMA sequence as in the canonical-A
// split launch, so C is bit-identical to it.  Needs N % 4 == 0 and
// 128 * N * 4 < 2^31 (the fp32 partial stores); the caller checks.
hipError_t launch_gemm_packed_splitk(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                     const uint8_t *b_s, int64_t M, int64_t N, int64_t K, void *c,
                                     bool c_bf16, const SplitPlan &sp, float *workspace, hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = workspace;
    p.M = M; p.N = N; p.K = K;
    p.KS = (int)packed_ksteps(K);
    p.NP = (int)packed_panels(N);
    p.G = 1;
    p.lda = K; p.lsa = K / 32; p.ldb = K; p.lsb = K / 32;
    p.tiles_m = (int)ceil_div(M, 256);
    p.tiles_n = (int)ceil_div(N, 128);
    p.splits = sp.splits;
    p.split_steps = sp.split_steps;
    p.c_stride = (M * N + 3) / 4 * 4;
    const int64_t units = (int64_t)p.tiles_m * p.tiles_n * sp.splits;
    dim3 grid((unsigned)std::min<int64_t>(units, device_cu_count())), block(kThreads);
    hipLaunchKernelGGL(gemm_ws_kernel<false>, grid, block, 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = M * N;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(n / 4, 256), 4096));
    if (c_bf16) hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                                   workspace, sp.splits, n, p.c_stride, c);
    else hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                            workspace, sp.splits, n, p.c_stride, c);
    return hipGetLastError();
}

// Accurate path: 256x128 tiles (dense, XCD-aware order), both operands
// staged in LDS as for mxfp8_gemm, each k-step computed by
// TileOps::acc_step.
hipError_t launch_gemm_accurate(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                const uint8_t *b_s, bool b_packed, int64_t M, int64_t N, int64_t K, void *c,
                                bool c_bf16, hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = c;
    p.M = M; p.N = N; p.K = K;
    p.KS = (int)packed_ksteps(K);
    p.NP = (int)packed_panels(N);
    p.G = 1;
    p.lda = K; p.lsa = K / 32; p.ldb = K; p.lsb = K / 32;
    p.tiles_m = (int)ceil_div(M, 256);
    p.tiles_n = (int)ceil_div(N, 128);
    dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(kThreads);
#define MX_ACC(BP, BF, KA) hipLaunchKernelGGL((gemm_kernel<256, 128, 4, BP, BF, false, KA, false, 2, false, true>), \
                                             grid, block, 0, stream, p)
    if (K % 128 == 0) {
        if (b_packed) { if (c_bf16) MX_ACC(true, true, true); else MX_ACC(true, false, true); }
        else { if (c_bf16) MX_ACC(false, true, true); else MX_ACC(false, false, true); }
    } else {
        if (b_packed) { if (c_bf16) MX_ACC(true, true, false); else MX_ACC(true, false, false); }
        else { if (c_bf16) MX_ACC(false, true, false); else MX_ACC(false, false, false); }
    }
#undef MX_ACC
    return hipGetLastError();
}

// Split-K plan for a dense GEMM on `cus` CUs: 256x128 tiles, as many K
// slices (each at least 4 k-steps) as keep tiles x slices within one round;
// splits == 1 means no split.
SplitPlan splitk_plan(int64_t M, int64_t N, int64_t K, int cus) {
    SplitPlan sp{1, (int)packed_ksteps(K), 0};
    const int64_t tiles = ceil_div(M, 256) * ceil_div(N, 128);
    const int64_t ks = packed_ksteps(K);
    if (tiles <= 0 || tiles * 2 > cus || ks < 8) return sp;
    int64_t s = cus / tiles;
    if (s > ks / 4) s = ks / 4;
    if (s < 2) return sp;
    const int64_t steps = ceil_div(ks, s);
    sp.splits = (int)ceil_div(ks, steps);      // every slice non-empty
    sp.split_steps = (int)steps;
    sp.workspace_bytes = (int64_t)sp.splits * ((M * N + 3) / 4 * 4) * 4;
    return sp;
}

hipError_t launch_gemm_splitk(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q, const uint8_t *b_s,
                              bool b_packed, int64_t M, int64_t N, int64_t K, void *c, bool c_bf16,
                              const SplitPlan &sp, float *workspace, hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = workspace;
    p.M = M; p.N = N; p.K = K;
    p.KS = (int)packed_ksteps(K);
    p.NP = (int)packed_panels(N);
    p.G = 1;
    p.lda = K; p.lsa = K / 32; p.ldb = K; p.lsb = K / 32;
    p.tiles_m = (int)ceil_div(M, 256);
    p.tiles_n = (int)ceil_div(N, 128);
    p.splits = sp.splits;
    p.split_steps = sp.split_steps;
    p.c_stride = (M * N + 3) / 4 * 4;
    dim3 grid((unsigned)(p.tiles_m * p.tiles_n * sp.splits)), block(kThreads);
    if (b_packed) hipLaunchKernelGGL(gemm_splitk_kernel<true>, grid, block, 0, stream, p);
    else hipLaunchKernelGGL(gemm_splitk_kernel<false>, grid, block, 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = M * N;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(n / 4, 256), 4096));
    if (c_bf16) hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                                   workspace, sp.splits, n, p.c_stride, c);
    else hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                            workspace, sp.splits, n, p.c_stride, c);
    return hipGetLastError();
}

// Grouped GEMM with packed A (the mxfp8_repack layout of the [M_total][K]
// rows): always the persistent 256-row launch (K % 128 == 0), whatever the
// group sizes; the same products per element as launch_grouped_gemm.
hipError_t launch_grouped_gemm_packed(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                      const uint8_t *b_s, const int32_t *offsets, int64_t G, int64_t M_total,
                                      int64_t N, int64_t K, void *c, bool c_bf16, hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = c;
    p.M = M_total; p.N = N; p.K = K;
    p.KS = (int)packed_ksteps(K);
    p.NP = (int)packed_panels(N);
    p.G = (int)G;
    p.offsets = offsets;
    p.lda = K; p.lsa = K / 32; p.ldb = K; p.lsb = K / 32;
    p.tiles_m = (int)(ceil_div(M_total, 256) + G);
    const int cus = device_cu_count();
    dim3 grid((unsigned)cus), block(kThreads);
    // the copying / computing-wave launch over 256x128 tiles while every
    // workgroup's share of the tiles (at most tiles_m x tiles_n of them, the
    // bound of each expert's ragged last tile) fits its tile table
    const int64_t ws_cols = ceil_div(N, 128);
    if (N % (c_bf16 ? 8 : 4) == 0 && (int64_t)128 * N * (c_bf16 ? 2 : 4) < ((int64_t)1 << 31) &&
        (int64_t)p.tiles_m * ws_cols <= (int64_t)(WsLayout::UNITS - 2) * cus) {
        p.tiles_n = (int)ws_cols;
        if (c_bf16) hipLaunchKernelGGL((gemm_ws_kernel<true, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((gemm_ws_kernel<false, true>), grid, block, 0, stream, p);
        return hipGetLastError();
    }
    p.tiles_n = (int)ceil_div(N, 256);
    if (c_bf16) hipLaunchKernelGGL((gemm_grouped_persist_kernel<true, false, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_grouped_persist_kernel<false, false, true>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// The experts' weight gradients with both operands packed along the token
// axis (K = T): the copying / computing-wave launch over (expert, tile) units,
// each over its expert's k-steps; an expert without tokens stores zeros.
hipError_t launch_grouped_gemm_wgrad_packed(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                            const uint8_t *b_s, const int32_t *offsets, int64_t G, int64_t T,
                                            int64_t M, int64_t N, void *c, bool c_bf16, hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = c;
    p.M = M; p.N = N; p.K = T;
    p.KS = (int)packed_ksteps(T);
    p.NP = (int)packed_panels(N);
    p.G = (int)G;
    p.offsets = offsets;
    p.c_stride = M * N;
    p.tiles_m = (int)ceil_div(M, 256);
    p.tiles_n = (int)ceil_div(N, 128);
    const int64_t units = G * p.tiles_m * p.tiles_n;
    dim3 grid((unsigned)std::min<int64_t>(units, device_cu_count())), block(kThreads);
    if (c_bf16) hipLaunchKernelGGL((gemm_ws_kernel<true, false, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_ws_kernel<false, false, true>), grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_wgrad(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                     const uint8_t *b_s, const int32_t *offsets, int64_t G,
                                     int64_t T, int64_t M, int64_t N, void *c, bool c_bf16,
                                     hipStream_t stream) {
    GemmParams p{};
    p.a_q = a_q; p.a_s = a_s; p.b_q = b_q; p.b_s = b_s; p.c = c;
    p.M = M; p.N = N; p.K = T;
    p.G = (int)G;
    p.offsets = offsets;
    p.lda = T; p.lsa = T / 32; p.ldb = T; p.lsb = T / 32;
    p.c_stride = M * N;
    constexpr int BM = 256, BN = 256;
    p.tiles_m = (int)ceil_div(M, BM);
    p.tiles_n = (int)ceil_div(N, BN);
    dim3 grid((unsigned)(G * p.tiles_m * p.tiles_n)), block(kThreads);
    if (T % 128 == 0) {
        if (c_bf16) hipLaunchKernelGGL(gemm_gk_aligned_kernel<true>, grid, block, 0, stream, p);
        else hipLaunchKernelGGL(gemm_gk_aligned_kernel<false>, grid, block, 0, stream, p);
    } else if (c_bf16) {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, 2, false, true, false, false, true>), grid, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, 2, false, false, false, false, true>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
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
    p.lda = K; p.lsa = K / 32; p.ldb = K; p.lsb = K / 32;
    // 256-row tiles move 1.0 operand byte per output per k-step against 1.5
    // for 128-row ones, but pad each group to 256 rows: they win once groups
    // average 256 rows (measured on the Qwen3-30B-A3B layer, 529 rows per
    // expert: gate_up 374 -> 340 us, down 279 -> 234 us)
    if (M_total >= 256 * G) {
        p.tiles_m = (int)(ceil_div(M_total, 256) + G);
        p.tiles_n = (int)ceil_div(N, 256);
        // persistent launch (measured on the Qwen3-30B-A3B layer: gate_up
        // 297 -> 282 us, down 214 -> 192 us against one workgroup per tile)
        if (K % 128 == 0) {
            dim3 grid((unsigned)device_cu_count()), block(kThreads);
            const bool sac = chunked_a_scales(K);
            if (sac) {
                if (c_bf16) hipLaunchKernelGGL((gemm_grouped_persist_kernel<true, true>), grid, block, 0, stream, p);
                else hipLaunchKernelGGL((gemm_grouped_persist_kernel<false, true>), grid, block, 0, stream, p);
            } else {
                if (c_bf16) hipLaunchKernelGGL((gemm_grouped_persist_kernel<true, false>), grid, block, 0, stream, p);
                else hipLaunchKernelGGL((gemm_grouped_persist_kernel<false, false>), grid, block, 0, stream, p);
            }
            return hipGetLastError();
        }
        return launch_tile<256, 256, 2, true>(p, true, c_bf16, p.tiles_m * p.tiles_n, stream);
    }
    p.tiles_m = (int)(ceil_div(M_total, 128) + G);
    p.tiles_n = (int)ceil_div(N, 256);
    return launch_tile<128, 256, 2, true>(p, true, c_bf16, p.tiles_m * p.tiles_n, stream);
}

}  // namespace mx
