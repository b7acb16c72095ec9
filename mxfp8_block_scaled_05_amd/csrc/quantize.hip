// MXFP8 quantizer kernels for gfx950.
//
// BF16 -> E4M3 elements + one E8M0 scale per 32-element block (page "End-to-End
// MXFP8 RL on Blackwell" (verl blog), section "The pipeline", paragraph "The
// format"; OCP MX v1.0 scale rule s = floor(log2 amax) - 8).  Both kernels are
// HBM-bound (3.03 algorithmic bytes per element: 2 in, 1 + 1/32 out); the
// design goal is full-width coalesced traffic with the arithmetic hidden.
//
//  - axis 1 (blocks along the contiguous axis): two lanes own one block,
//    16 BF16 (32 B) each, so a wave's q store is a contiguous 1 KB.  The block
//    max is an integer max over BF16 magnitude bits, completed across the
//    lane pair with one DPP quad permute (no LDS).  Elements are scaled by an
//    exact power of two, clamped to +-448 and converted with the hardware
//    E4M3 conversion (round to nearest even).  A fixed set of waves walks the
//    array with the next step's loads in flight.
//  - axis 0 (blocks along rows, output transposed): a workgroup owns a
//    128-row x 128-column tile and transposes it through LDS, so global loads
//    are 16-byte row reads and global stores whole 128-byte output lines;
//    each lane reduces and converts its column's block in registers.
//  - both axes from one read (learner tensors), and weights quantized straight
//    into the GEMM's packed layout (weight sync), share the LDS tile code.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ us2 as_us2(uint32_t v) { return __builtin_bit_cast(us2, v); }
__device__ __forceinline__ uint32_t as_u32(us2 v) { return __builtin_bit_cast(uint32_t, v); }

// max of the two BF16 magnitudes packed in each dword, over n dwords
__device__ __forceinline__ uint32_t max_mag(const uint32_t *d, int n) {
    us2 m = as_us2(d[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < n; ++i) m = __builtin_elementwise_max(m, as_us2(d[i] & 0x7FFF7FFFu));
    return m.x > m.y ? m.x : m.y;
}

// Four dwords (8 BF16) -> two dwords (8 E4M3) with the block's inverse scale.
__device__ __forceinline__ v2i convert8(const uint32_t *d, float inv) {
    v2i out;
    int w0 = cvt2_e4m3<false>(bits_to_float(d[0] << 16) * inv,
                              bits_to_float(d[0] & 0xFFFF0000u) * inv, 0);
    w0 = cvt2_e4m3<true>(bits_to_float(d[1] << 16) * inv,
                         bits_to_float(d[1] & 0xFFFF0000u) * inv, w0);
    int w1 = cvt2_e4m3<false>(bits_to_float(d[2] << 16) * inv,
                              bits_to_float(d[2] & 0xFFFF0000u) * inv, 0);
    w1 = cvt2_e4m3<true>(bits_to_float(d[3] << 16) * inv,
                         bits_to_float(d[3] & 0xFFFF0000u) * inv, w1);
    out.x = w0;
    out.y = w1;
    return out;
}

// quad_perm DPP control [1,0,3,2]: swap the lanes of each pair
constexpr int kQuadSwap1 = 0xB1;
// The axis-1 quantizer's strided walk: resident waves per CU, and the input
// size from which its loads and stores are nontemporal.  Measured on MI355X
// (settled clocks, medians): 32 waves per CU instead of 16 take 6144x4096
// from 16.5 to 16.0 us and 4096x4096 from 12.3 to 11.5 us (more bytes in
// flight while the launch ramps up); nontemporal accesses take 8192x24576 and
// 16384x16384 from 5.2-5.35 to 5.46 TB/s but slow the tensors that fit the
// 256 MB Infinity Cache (6144x4096: 16.5 -> 18.1 us), so only inputs of at
// least that size use them, with 16 waves per CU.
constexpr int kQuantWavesPerCu = 32;
constexpr int kQuantWavesPerCuLarge = 16;
constexpr int64_t kQuantNontemporalBytes = 256ll << 20;
// resident waves per CU of the gather quantizer (the axis-1 walk over gathered rows)
constexpr int kGatherWavesPerCu = 16;

// ---------------------------------------------------------------- axis 1
// The flat array of blocks (rows * cols / 32 of them; a block never straddles
// a row because cols % 32 == 0) is cut into wave-steps of 64 blocks (4 KB of
// BF16): sub-step h in {0, 1} covers blocks 32h .. 32h+31, lane l the half
// l % 2 of block 32h + l/2, loaded as two 16-byte pieces (d[2h], d[2h+1]).
// Each wave walks a strided list of steps with the next step's loads in
// flight while it converts the current one, so a wave pays the memory latency
// once, not once per step.
template <bool NT = false>
__device__ __forceinline__ void load_step(const uint16_t *__restrict__ x, int64_t b0,
                                          int64_t nblocks, int lane, uint32_t (*d)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t blk = b0 + (u >> 1) * 32 + (lane >> 1);
        if (blk < nblocks) {
            const v4i *p = reinterpret_cast<const v4i *>(x + blk * 32 + (lane & 1) * 16 + (u & 1) * 8);
            const v4i v = NT ? __builtin_nontemporal_load(p) : *p;
            d[u][0] = v.x; d[u][1] = v.y; d[u][2] = v.z; d[u][3] = v.w;
        } else {
            d[u][0] = d[u][1] = d[u][2] = d[u][3] = 0;
        }
    }
}

template <bool NT = false>
__device__ __forceinline__ void convert_step(uint8_t *__restrict__ q, uint8_t *__restrict__ scales,
                                             int64_t b0, int64_t nblocks, int lane,
                                             uint32_t (*d)[4]) {
    uint32_t code[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t m = max(max_mag(d[2 * h], 4), max_mag(d[2 * h + 1], 4));
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadSwap1, 0xF, 0xF, false));
        code[h] = scale_code_from_amax_bits(m);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t blk = b0 + h * 32 + (lane >> 1);
        const float inv = inv_scale_from_code(code[h]);
        v2i o0 = convert8(d[2 * h], inv), o1 = convert8(d[2 * h + 1], inv);
        v4i o = v4i{o0.x, o0.y, o1.x, o1.y};
        if (code[h] == 255u) o = v4i{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
        if (blk < nblocks) {
            v4i *p = reinterpret_cast<v4i *>(q + blk * 32 + (lane & 1) * 16);
            if constexpr (NT) __builtin_nontemporal_store(o, p);
            else *p = o;
        }
    }
    // lane l stores the scale of block b0 + l, held by lane 2*(l%32) of sub-step l/32
    const int src = (lane & 31) * 2;
    const uint32_t s0 = __shfl(code[0], src), s1 = __shfl(code[1], src);
    const uint32_t sc = lane < 32 ? s0 : s1;
    if (b0 + lane < nblocks) scales[b0 + lane] = (uint8_t)sc;
}

template <bool NT>
__global__ __launch_bounds__(256) void quantize_axis1_kernel(const uint16_t *__restrict__ x,
                                                             uint8_t *__restrict__ q,
                                                             uint8_t *__restrict__ scales,
                                                             int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t nsteps = (nblocks + 63) / 64;
    int64_t step = wave;
    if (step >= nsteps) return;
    uint32_t cur[4][4], nxt[4][4];
    load_step<NT>(x, step * 64, nblocks, lane, cur);
    for (; step < nsteps; step += nwaves) {
        const bool more = step + nwaves < nsteps;
        if (more) load_step<NT>(x, (step + nwaves) * 64, nblocks, lane, nxt);
        convert_step<NT>(q, scales, step * 64, nblocks, lane, cur);
        if (more) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) cur[u][k] = nxt[u][k];
        }
    }
}

// The same walk writing the packed layout (the GEMM's operand layout, as
// mxfp8_repack defines it): a step is one 16-row atom x one 128-column k-step
// (64 blocks, 4 KB of BF16 as above), atom-major, over every atom of every
// 256-row panel.  Sub-step h covers the atom's rows 8h .. 8h+7: lane l holds
// half l % 2 of block (l / 2) % 4 of row 8h + l / 8, loaded as two 16-byte
// pieces.  The step's codes are 16 rows x 128 bytes of one packed tile (each
// row's 16-byte chunk c at slot c ^ (row % 8)), its 64 scale bytes the atom's
// 64-byte per-lane record of that k-step; rows past `rows` and blocks past
// cols / 32 are written as the layout's padding (codes 0, scale 127).
// (steps of a packed job < 2^31, so the step index math is 32-bit)
__device__ __forceinline__ void load_step_packed(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                                                 int KS, int st, int lane, uint32_t (*d)[4]) {
    const int atom = st / KS, ks = st - atom * KS;
    const int bl = lane >> 1, half = lane & 1, i = bl >> 2, kb4 = bl & 3;
    const int kcol = ks * (int)kKStep + kb4 * 32 + half * 16;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t r = (int64_t)atom * 16 + (u >> 1) * 8 + i;
        const int k = kcol + (u & 1) * 8;
        if (r < rows && k < cols) {
            const v4i v = *reinterpret_cast<const v4i *>(x + r * cols + k);
            d[u][0] = v.x; d[u][1] = v.y; d[u][2] = v.z; d[u][3] = v.w;
        } else {
            d[u][0] = d[u][1] = d[u][2] = d[u][3] = 0;
        }
    }
}

__device__ __forceinline__ void convert_step_packed(uint8_t *__restrict__ qp, uint8_t *__restrict__ sp,
                                                    int64_t rows, int64_t cols, int KS, int st,
                                                    int lane, uint32_t (*d)[4]) {
    const int atom = st / KS, ks = st - atom * KS;
    const int bl = lane >> 1, half = lane & 1, i = bl >> 2, kb4 = bl & 3;
    const bool kvalid = ks * 4 + kb4 < (int)(cols / 32);
    const int64_t tile_lin = (int64_t)(atom >> 4) * KS + ks;
    const int arow0 = (atom & 15) * 16;
    uint32_t code[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t m = max(max_mag(d[2 * h], 4), max_mag(d[2 * h + 1], 4));
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadSwap1, 0xF, 0xF, false));
        const bool valid = kvalid && (int64_t)atom * 16 + h * 8 + i < rows;
        code[h] = valid ? scale_code_from_amax_bits(m) : 127u;
    }
    uint8_t *qtile = qp + tile_lin * kTileBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float inv = inv_scale_from_code(code[h]);
        v2i o0 = convert8(d[2 * h], inv), o1 = convert8(d[2 * h + 1], inv);
        v4i o = v4i{o0.x, o0.y, o1.x, o1.y};
        if (code[h] == 255u) o = v4i{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
        const int rp = arow0 + h * 8 + i;              // row inside the panel
        const int c = kb4 * 2 + half;                  // 16-byte chunk of the row's 128 bytes
        *reinterpret_cast<v4i *>(qtile + rp * 128 + ((c ^ (int)swz((uint32_t)rp)) << 4)) = o;
    }
    // lane l stores the scale of row l % 16, block l / 16 of the step: held by
    // lane 2 * (4 * (row % 8) + block) of sub-step row / 8
    const int rr = lane & 15, src = 2 * ((rr & 7) * 4 + (lane >> 4));
    const uint32_t s0 = __shfl(code[0], src), s1 = __shfl(code[1], src);
    sp[tile_lin * kScaleStepBytes + (atom & 15) * 64 + lane] = (uint8_t)(rr < 8 ? s0 : s1);
}

// Several tensors in one launch: the wave-steps of tensor i are
// step_end[i-1] .. step_end[i]-1 of one index space that the waves walk as
// above; each step finds its tensor from the running step totals (uniform over
// the wave, so the table is read by scalar loads).
__device__ __forceinline__ int quant_job_of(const QuantJobs &jobs, int64_t step) {
    int j = 0;
#pragma unroll
    for (int i = 0; i < kQuantJobsMax - 1; ++i)
        if (i < jobs.count - 1 && step >= jobs.step_end[i]) j = i + 1;
    return j;
}

// PACKED: some jobs write the packed layout.  That step needs about 18 more
// registers, so it is a variant of its own, launched with 6 workgroups per CU;
// a list of canonical jobs only keeps the leaner variant at 8 per CU.
template <bool PACKED>
__global__ __launch_bounds__(256) void quantize_axis1_many_kernel(QuantJobs jobs) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t nsteps = jobs.step_end[jobs.count - 1];
    int64_t step = wave;
    if (step >= nsteps) return;
    uint32_t cur[4][4], nxt[4][4];
    // a step of job jj, local index st, into registers d (the job is uniform
    // over the wave, so the branch on its layout is too)
    auto load = [&](int jj, int64_t st, uint32_t (*d)[4]) {
        if (PACKED && jobs.packed[jj])
            load_step_packed(jobs.x[jj], jobs.rows[jj], jobs.cols[jj], (int)((jobs.cols[jj] + kKStep - 1) / kKStep),
                             (int)st, lane, d);
        else
            load_step(jobs.x[jj], st * 64, jobs.nblocks[jj], lane, d);
    };
    int j = quant_job_of(jobs, step);
    load(j, step - (j ? jobs.step_end[j - 1] : 0), cur);
    for (; step < nsteps; step += nwaves) {
        const bool more = step + nwaves < nsteps;
        int jn = j;
        if (more) {
            jn = quant_job_of(jobs, step + nwaves);
            load(jn, step + nwaves - (jn ? jobs.step_end[jn - 1] : 0), nxt);
        }
        const int64_t st = step - (j ? jobs.step_end[j - 1] : 0);
        if (PACKED && jobs.packed[j])
            convert_step_packed(jobs.q[j], jobs.s[j], jobs.rows[j], jobs.cols[j],
                                (int)((jobs.cols[j] + kKStep - 1) / kKStep), (int)st, lane, cur);
        else
            convert_step(jobs.q[j], jobs.s[j], st * 64, jobs.nblocks[j], lane, cur);
        if (more) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) cur[u][k] = nxt[u][k];
        }
        j = jn;
    }
}

// ---------------------------------------------------------------- tiles in LDS
// A 128-column BF16 tile in LDS: row r (256 B) holds its 16-byte chunk c at
// slot c ^ (r % 16).  Column-pair dword reads (64 lanes over one row) and
// block reads (a lane reads chunks 4b..4b+3 of its own row, 16 lanes over 4
// rows x 4 blocks or 16 rows x 1 block) both hit 16 distinct chunk slots, so
// neither has bank conflicts.
__device__ __forceinline__ int tile_slot(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

// BF16 rows [R0, R0 + nrows) x columns [C0, C0 + 128) of x[rows][cols] into the
// tile (zeros outside the matrix).  256 threads.
template <int NROWS>
__device__ __forceinline__ void load_tile(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                                          int64_t R0, int64_t C0, uint8_t *tile, int t) {
    if ((cols & 7) == 0) {
        // rows are 16-byte aligned: sixteen 16-byte chunks per tile row
        const int ch = t & 15;
        const int64_t c = C0 + ch * 8;
#pragma unroll
        for (int i = 0; i < NROWS / 16; ++i) {
            const int r = i * 16 + (t >> 4);
            v4i v = v4i{0, 0, 0, 0};
            if (R0 + r < rows && c < cols) v = *reinterpret_cast<const v4i *>(x + (R0 + r) * cols + c);
            *reinterpret_cast<v4i *>(tile + tile_slot(r, ch)) = v;
        }
    } else {
        for (int i = t; i < NROWS * 64; i += 256) {
            const int r = i >> 6, cp = i & 63;
            const int64_t row = R0 + r, c = C0 + 2 * cp;
            uint32_t v = 0;
            if (row < rows) {
                if (c < cols) v = x[row * cols + c];
                if (c + 1 < cols) v |= (uint32_t)x[row * cols + c + 1] << 16;
            }
            *reinterpret_cast<uint32_t *>(tile + tile_slot(r, cp >> 2) + (cp & 3) * 4) = v;
        }
    }
}

// Quantize block b (columns 32b .. 32b+31) of tile row r: scale code and the
// 32 E4M3 bytes as 8 dwords (NaN/Inf blocks: code 0xFF, elements 0x7F).
__device__ __forceinline__ uint32_t quantize_row_block(const uint8_t *tile, int r, int b, uint32_t *q8) {
    uint32_t d[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const v4i v = *reinterpret_cast<const v4i *>(tile + tile_slot(r, 4 * b + j));
        d[4 * j] = v.x; d[4 * j + 1] = v.y; d[4 * j + 2] = v.z; d[4 * j + 3] = v.w;
    }
    const uint32_t code = scale_code_from_amax_bits(max_mag(d, 16));
    const float inv = inv_scale_from_code(code);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const v2i o = convert8(d + 4 * j, inv);
        q8[2 * j] = code == 255u ? 0x7F7F7F7Fu : (uint32_t)o.x;
        q8[2 * j + 1] = code == 255u ? 0x7F7F7F7Fu : (uint32_t)o.y;
    }
    return code;
}

// ---------------------------------------------------------------- gather + axis 1
// Routing permute fused with the quantizer: output row i is input row
// idx[i] (a row index outside [0, rows_in) -- the padding of an expert group
// -- gives a zero row), quantized along its columns.  The same wave-step walk
// as quantize_axis1_kernel over the output's blocks; a block never straddles
// a row, so each lane pair reads one contiguous 64-byte block of its source
// row.
__device__ __forceinline__ void load_step_gather(const uint16_t *__restrict__ x, int64_t rows_in,
                                                 int64_t bpr, const int64_t *__restrict__ idx,
                                                 int64_t b0, int64_t nblocks, int lane,
                                                 uint32_t (*d)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t blk = b0 + (u >> 1) * 32 + (lane >> 1);
        d[u][0] = d[u][1] = d[u][2] = d[u][3] = 0;
        if (blk < nblocks) {
            const int64_t src = idx[blk / bpr];
            if (src >= 0 && src < rows_in) {
                const v4i v = *reinterpret_cast<const v4i *>(x + (src * bpr + blk % bpr) * 32 +
                                                            (lane & 1) * 16 + (u & 1) * 8);
                d[u][0] = v.x; d[u][1] = v.y; d[u][2] = v.z; d[u][3] = v.w;
            }
        }
    }
}

__global__ __launch_bounds__(256) void quantize_gather_kernel(const uint16_t *__restrict__ x,
                                                              int64_t rows_in, int64_t bpr,
                                                              const int64_t *__restrict__ idx,
                                                              uint8_t *__restrict__ q,
                                                              uint8_t *__restrict__ scales,
                                                              int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t nsteps = (nblocks + 63) / 64;
    int64_t step = wave;
    if (step >= nsteps) return;
    uint32_t cur[4][4], nxt[4][4];
    load_step_gather(x, rows_in, bpr, idx, step * 64, nblocks, lane, cur);
    for (; step < nsteps; step += nwaves) {
        const bool more = step + nwaves < nsteps;
        if (more) load_step_gather(x, rows_in, bpr, idx, (step + nwaves) * 64, nblocks, lane, nxt);
        convert_step(q, scales, step * 64, nblocks, lane, cur);
        if (more) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) cur[u][k] = nxt[u][k];
        }
    }
}

// Gather + axis 1 straight into the packed layout (N = rows_out, K = cols):
// the atom walk of the list quantizer's packed jobs (a wave-step is 16 rows
// by one 128-column k-step), each output row read from x[idx[row]] (an index
// outside [0, rows_in) gives a zero row); atoms and blocks past the matrix
// write the layout's padding.
__device__ __forceinline__ void load_step_packed_gather(const uint16_t *__restrict__ x, int64_t rows_in, int64_t cols,
                                                        const int64_t *__restrict__ idx, int64_t rows_out, int KS,
                                                        int st, int lane, uint32_t (*d)[4]) {
    const int atom = st / KS, ks = st - atom * KS;
    const int bl = lane >> 1, half = lane & 1, i = bl >> 2, kb4 = bl & 3;
    const int kcol = ks * (int)kKStep + kb4 * 32 + half * 16;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t r = (int64_t)atom * 16 + (u >> 1) * 8 + i;
        const int k = kcol + (u & 1) * 8;
        const int64_t src = r < rows_out ? idx[r] : -1;
        if (src >= 0 && src < rows_in && k < cols) {
            const v4i v = *reinterpret_cast<const v4i *>(x + src * cols + k);
            d[u][0] = v.x; d[u][1] = v.y; d[u][2] = v.z; d[u][3] = v.w;
        } else {
            d[u][0] = d[u][1] = d[u][2] = d[u][3] = 0;
        }
    }
}

__global__ __launch_bounds__(256) void quantize_gather_packed_kernel(const uint16_t *__restrict__ x,
                                                                     int64_t rows_in, int64_t cols,
                                                                     const int64_t *__restrict__ idx,
                                                                     int64_t rows_out, uint8_t *__restrict__ qp,
                                                                     uint8_t *__restrict__ sp, int64_t nsteps) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int KS = (int)((cols + kKStep - 1) / kKStep);
    int64_t step = wave;
    if (step >= nsteps) return;
    uint32_t cur[4][4], nxt[4][4];
    load_step_packed_gather(x, rows_in, cols, idx, rows_out, KS, (int)step, lane, cur);
    for (; step < nsteps; step += nwaves) {
        const bool more = step + nwaves < nsteps;
        if (more) load_step_packed_gather(x, rows_in, cols, idx, rows_out, KS, (int)(step + nwaves), lane, nxt);
        convert_step_packed(qp, sp, rows_out, cols, KS, (int)step, lane, cur);
        if (more) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) cur[u][k] = nxt[u][k];
        }
    }
}

// ---------------------------------------------------------------- axis 0
// x[rows][cols] -> q[cols][rows], scales[cols][rows/32].  A workgroup of four
// waves owns a 128-row x 128-column tile and moves it through LDS twice:
//   1. the BF16 tile is read with 16-byte row loads into LDS,
//   2. wave w takes rows [32w, 32w+32), lane l the column pair (2l, 2l+1): it
//      reads its two 32-element blocks as 32 dwords and quantizes them in
//      registers,
//   3. the E4M3 tile is written back to the same LDS as [128 columns][128 B]
//      (padded rows) and stored to q as whole 128-byte lines.
constexpr int kA0Tile = 128;
constexpr int kA0OutPitch = 144;  // bytes per staged output column (16-byte aligned)

// Step 2: the tile's 128 columns quantized along its rows into the staging
// area: column c's 128 codes at tile + c * kA0OutPitch (16-byte chunk j holds
// rows 16j..16j+15), its four scale codes at stile[c * 4 + b] (block b = rows
// 32b..32b+31).  Ends with a barrier; the staged tile is then ready to store.
__device__ __forceinline__ void axis0_stage_tile(uint8_t *tile, uint8_t *stile, int t) {
    const int lane = t & 63, w = t >> 6;
    uint32_t d[32];
#pragma unroll
    for (int r = 0; r < 32; ++r)
        d[r] = *reinterpret_cast<const uint32_t *>(tile + tile_slot(32 * w + r, lane >> 2) + (lane & 3) * 4);
    __syncthreads();  // the tile is reused for the output below

    us2 m = as_us2(d[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int r = 1; r < 32; ++r) m = __builtin_elementwise_max(m, as_us2(d[r] & 0x7FFF7FFFu));
    const uint32_t code_lo = scale_code_from_amax_bits(m.x);
    const uint32_t code_hi = scale_code_from_amax_bits(m.y);
    const float inv_lo = inv_scale_from_code(code_lo);
    const float inv_hi = inv_scale_from_code(code_hi);
    uint8_t *ob = tile;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int wl[4], wh[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = h * 16 + k * 4;
            int a = cvt2_e4m3<false>(bits_to_float(d[r] << 16) * inv_lo,
                                     bits_to_float(d[r + 1] << 16) * inv_lo, 0);
            wl[k] = cvt2_e4m3<true>(bits_to_float(d[r + 2] << 16) * inv_lo,
                                    bits_to_float(d[r + 3] << 16) * inv_lo, a);
            int b = cvt2_e4m3<false>(bits_to_float(d[r] & 0xFFFF0000u) * inv_hi,
                                     bits_to_float(d[r + 1] & 0xFFFF0000u) * inv_hi, 0);
            wh[k] = cvt2_e4m3<true>(bits_to_float(d[r + 2] & 0xFFFF0000u) * inv_hi,
                                    bits_to_float(d[r + 3] & 0xFFFF0000u) * inv_hi, b);
        }
        v4i lo = v4i{wl[0], wl[1], wl[2], wl[3]};
        v4i hi = v4i{wh[0], wh[1], wh[2], wh[3]};
        if (code_lo == 255u) lo = v4i{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
        if (code_hi == 255u) hi = v4i{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
        *reinterpret_cast<v4i *>(ob + (2 * lane) * kA0OutPitch + 32 * w + 16 * h) = lo;
        *reinterpret_cast<v4i *>(ob + (2 * lane + 1) * kA0OutPitch + 32 * w + 16 * h) = hi;
    }
    stile[(2 * lane) * 4 + w] = (uint8_t)code_lo;
    stile[(2 * lane + 1) * 4 + w] = (uint8_t)code_hi;
    __syncthreads();
}

// Steps 2 and 3 for one tile already in LDS (`tile`, reused for the output).
// dstb (optional, in LDS): destination 32-row block in an output of rows_out
// rows for each of the tile's four source blocks (-1: not written); without
// it block b goes to block R0/32 + b of an output of `rows` rows.
__device__ __forceinline__ void axis0_from_tile(uint8_t *tile, uint8_t *stile, uint8_t *__restrict__ q,
                                                uint8_t *__restrict__ scales, int64_t rows, int64_t cols,
                                                int64_t R0, int64_t C0, int t, const int *dstb = nullptr,
                                                int64_t rows_out = 0) {
    axis0_stage_tile(tile, stile, t);
    const uint8_t *ob = tile;
    if (dstb != nullptr) {
        // regrouped output: each 16-byte chunk lies in one 32-row block
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = i * 32 + (t >> 3), j = t & 7;
            const int64_t c = C0 + col;
            const int d = dstb[j >> 1];
            if (c < cols && d >= 0)
                *reinterpret_cast<v4i *>(q + c * rows_out + (int64_t)d * 32 + 16 * (j & 1)) =
                    *reinterpret_cast<const v4i *>(ob + col * kA0OutPitch + 16 * j);
        }
        if (t < kA0Tile && C0 + t < cols) {
            uint8_t *srow = scales + (C0 + t) * (rows_out / 32);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (dstb[b] >= 0) srow[dstb[b]] = stile[t * 4 + b];
        }
        return;
    }
    // eight lanes store one output column's 128-byte line; rows % 32 == 0, so a
    // 16-byte chunk of the line is either wholly inside the matrix or outside
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = i * 32 + (t >> 3), j = t & 7;
        const int64_t c = C0 + col, r = R0 + 16 * j;
        if (c < cols && r < rows)
            *reinterpret_cast<v4i *>(q + c * rows + r) =
                *reinterpret_cast<const v4i *>(ob + col * kA0OutPitch + 16 * j);
    }
    const int64_t nb = rows / 32;
    if (t < kA0Tile && C0 + t < cols) {
        uint8_t *srow = scales + (C0 + t) * nb + R0 / 32;
        if ((nb & 3) == 0 && R0 + kA0Tile <= rows) {
            // the tile's four scales of this column are one aligned dword
            *reinterpret_cast<uint32_t *>(srow) = reinterpret_cast<const uint32_t *>(stile)[t];
        } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (R0 + 32 * b < rows) srow[b] = stile[t * 4 + b];
        }
    }
}

// The regrouped axis-0 grid straight into the packed layout of the weight
// gradient's operand (N = cols, K = rows_out): destination 32-row block d of
// column f is K-block d % 4 of k-step d / 4 of row f % 256 of panel f / 256,
// its two 16-byte chunks at slots c ^ (f % 8), its scale byte at the panel
// row's place in the step's scale tile -- what mxfp8_repack writes for the
// canonical regrouped grid.
__device__ __forceinline__ void axis0_from_tile_packed(uint8_t *tile, uint8_t *stile, uint8_t *__restrict__ qp,
                                                       uint8_t *__restrict__ sp, int64_t cols, int64_t C0, int t,
                                                       const int *dstb, int64_t KS) {
    axis0_stage_tile(tile, stile, t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = i * 32 + (t >> 3), j = t & 7;
        const int64_t f = C0 + col;
        const int d = dstb[j >> 1];
        if (f < cols && d >= 0) {
            const int64_t tl = (f / kPanelRows) * KS + d / 4;
            const int frow = (int)(f % kPanelRows), c = 2 * (d & 3) + (j & 1);
            *reinterpret_cast<v4i *>(qp + tl * kTileBytes + frow * kKStep + ((c ^ (frow & 7)) << 4)) =
                *reinterpret_cast<const v4i *>(tile + col * kA0OutPitch + 16 * j);
        }
    }
    if (t < kA0Tile && C0 + t < cols) {
        const int64_t f = C0 + t;
        const int frow = (int)(f % kPanelRows);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int d = dstb[b];
            if (d >= 0)
                sp[((f / kPanelRows) * KS + d / 4) * kScaleStepBytes + (frow >> 4) * 64 + (frow & 15) + 16 * (d & 3)] =
                    stile[t * 4 + b];
        }
    }
}

// one workgroup per tile; tiles numbered row-tile-major over a 1-D grid
// (batched: matrix-major)
__device__ __forceinline__ void tile_origin_of(int64_t idx, int64_t rows, int64_t cols, int64_t &b, int64_t &R0,
                                               int64_t &C0) {
    const int64_t tiles_c = (cols + kA0Tile - 1) / kA0Tile;
    const int64_t tiles = ((rows + kA0Tile - 1) / kA0Tile) * tiles_c;
    const int64_t t = idx % tiles;
    b = idx / tiles;
    R0 = (t / tiles_c) * kA0Tile;
    C0 = (t % tiles_c) * kA0Tile;
}
__device__ __forceinline__ void tile_origin(int64_t rows, int64_t cols, int64_t &b, int64_t &R0,
                                            int64_t &C0) {
    tile_origin_of(blockIdx.x, rows, cols, b, R0, C0);
}

// The tile walk used when cols % 8 == 0: a workgroup takes tiles blockIdx.x,
// blockIdx.x + gridDim.x, ... and keeps the next tile's sixteen-byte loads in
// registers (in flight) while it quantizes the current one out of LDS, so the
// load latency of a tile overlaps the previous tile's work.
// NT: nontemporal loads (measured on MI355X: axis 0 on 16384x16384 4.24 ->
// 5.18 TB/s and 6144x4096 20.1 -> 18.9 us; both axes on 8192x24576 4.34 ->
// 4.49 TB/s but 4096x4096 18.1 -> 20.2 us, so both axes take them only for
// inputs of at least the Infinity Cache's size).  Nontemporal stores on top
// of them: axis 0 on 16384x16384 5.32 -> 4.30 TB/s, both axes unchanged, so
// the stores stay plain.
constexpr int kA0Loads = kA0Tile / 16;     // 16-byte loads per thread per tile
template <bool NT>
__device__ __forceinline__ void load_tile_regs(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                                               int64_t R0, int64_t C0, int t, v4i *v) {
    const int ch = t & 15;
    const int64_t c = C0 + ch * 8;
#pragma unroll
    for (int i = 0; i < kA0Loads; ++i) {
        const int r = i * 16 + (t >> 4);
        v[i] = v4i{0, 0, 0, 0};
        if (R0 + r < rows && c < cols) {
            const v4i *p = reinterpret_cast<const v4i *>(x + (R0 + r) * cols + c);
            v[i] = NT ? __builtin_nontemporal_load(p) : *p;
        }
    }
}
__device__ __forceinline__ void store_tile_regs(uint8_t *tile, int t, const v4i *v) {
    const int ch = t & 15;
#pragma unroll
    for (int i = 0; i < kA0Loads; ++i)
        *reinterpret_cast<v4i *>(tile + tile_slot(i * 16 + (t >> 4), ch)) = v[i];
}

// x[batch][rows][cols] -> q[batch][cols][rows], scales[batch][cols][rows/32]
__global__ __launch_bounds__(256) void quantize_axis0_kernel(const uint16_t *__restrict__ x,
                                                             uint8_t *__restrict__ q,
                                                             uint8_t *__restrict__ scales,
                                                             int64_t rows, int64_t cols) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kA0Tile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kA0Tile * 4];
    static_assert(kA0Tile * kA0OutPitch <= (int)sizeof(tile), "output stage fits the input stage");
    int64_t b, R0, C0;
    tile_origin(rows, cols, b, R0, C0);
    load_tile<kA0Tile>(x + b * rows * cols, rows, cols, R0, C0, tile, threadIdx.x);
    __syncthreads();
    axis0_from_tile(tile, stile, q + b * rows * cols, scales + b * cols * (rows / 32), rows, cols, R0,
                    C0, threadIdx.x);
}

// ---------------------------------------------------------------- both axes
// One BF16 read, both operand grids of a learner tensor (rows % 32 == 0 and
// cols % 32 == 0): the tile in LDS is first quantized along its rows (axis 1:
// 512 blocks, two per thread, each lane's 32 output bytes part of a 128-byte
// row segment), then along its columns exactly as the axis-0 kernel does.
// 4.0625 algorithmic bytes per element instead of 2 x 3.03125.
__global__ __launch_bounds__(256) void quantize_dual_kernel(const uint16_t *__restrict__ x,
                                                            uint8_t *__restrict__ q_row,
                                                            uint8_t *__restrict__ s_row,
                                                            uint8_t *__restrict__ q_col,
                                                            uint8_t *__restrict__ s_col,
                                                            int64_t rows, int64_t cols) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kA0Tile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kA0Tile * 4];
    const int t = threadIdx.x;
    int64_t b_unused, R0, C0;
    tile_origin(rows, cols, b_unused, R0, C0);
    load_tile<kA0Tile>(x, rows, cols, R0, C0, tile, t);
    __syncthreads();
    const int64_t nb = cols / 32;
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
        const int u = u2 * 256 + t, r = u >> 2, b = u & 3;
        uint32_t q8[8];
        const uint32_t code = quantize_row_block(tile, r, b, q8);
        const int64_t row = R0 + r, c = C0 + 32 * b;
        if (row < rows && c < cols) {
            v4i *dst = reinterpret_cast<v4i *>(q_row + row * cols + c);
            dst[0] = v4i{(int)q8[0], (int)q8[1], (int)q8[2], (int)q8[3]};
            dst[1] = v4i{(int)q8[4], (int)q8[5], (int)q8[6], (int)q8[7]};
            s_row[row * nb + c / 32] = (uint8_t)code;
        }
    }
    axis0_from_tile(tile, stile, q_col, s_col, rows, cols, R0, C0, t);
}

// ---------------------------------------------------------------- regrouped axis 0
// Row (token) regrouping of the axis-0 output: group g's source rows
// [s_g, s_g+1) go to output rows [d_g, d_g + (s_g+1 - s_g)) of an output with
// rows_out rows; the rest of [d_g, d_g+1) is zero (pad).  Offsets are read on
// the device and clamped like the grouped GEMM's ([0, rows] and [0, rows_out],
// each range at least empty), so a malformed table can only drop rows; a
// source block goes nowhere unless its group's source and destination starts
// are multiples of 32 and the block fits inside the group's destination range.

// Wave-wide search: the first group g whose clamped source range holds row
// `row`; returns g (or -1) and that group's clamped source start.
__device__ int find_src_group(const int32_t *src_off, int G, int64_t rows, int64_t row, int lane, int64_t &lo) {
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        int64_t l = 0, h = 0;
        if (g < G) {
            l = src_off[g];
            h = src_off[g + 1];
            l = l < 0 ? 0 : (l > rows ? rows : l);
            h = h < l ? l : (h > rows ? rows : h);
        }
        const unsigned long long hit = __ballot(g < G && row >= l && row < h);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            lo = __shfl(l, src);
            return g0 + src;
        }
    }
    return -1;
}

// destination block of the source block starting at row `row`, or -1
__device__ int dst_block_of(const int32_t *src_off, const int32_t *dst_off, int G, int64_t rows,
                            int64_t rows_out, int64_t row, int lane) {
    if (row >= rows) return -1;
    int64_t lo;
    const int g = find_src_group(src_off, G, rows, row, lane, lo);
    if (g < 0) return -1;
    int64_t dlo = dst_off[g], dhi = dst_off[g + 1];
    dlo = dlo < 0 ? 0 : (dlo > rows_out ? rows_out : dlo);
    dhi = dhi < dlo ? dlo : (dhi > rows_out ? rows_out : dhi);
    if ((lo & 31) || (dlo & 31)) return -1;
    const int64_t d = dlo + (row - lo);
    return d + 32 <= dhi ? (int)(d / 32) : -1;
}

// both axes of x[rows][cols]: axis 1 (optional) as quantize_dual_kernel, axis
// 0 regrouped into q_col[cols][rows_out], s_col[cols][rows_out/32]
__global__ __launch_bounds__(256) void quantize_dual_grouped_kernel(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q_row, uint8_t *__restrict__ s_row,
    uint8_t *__restrict__ q_col, uint8_t *__restrict__ s_col, int64_t rows, int64_t cols,
    const int32_t *__restrict__ src_off, const int32_t *__restrict__ dst_off, int G, int64_t rows_out) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kA0Tile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kA0Tile * 4];
    __shared__ int dstb[4];
    const int t = threadIdx.x;
    int64_t b_unused, R0, C0;
    tile_origin(rows, cols, b_unused, R0, C0);
    {
        // wave w finds the destination of the tile's source block w
        const int w = t >> 6;
        const int d = dst_block_of(src_off, dst_off, G, rows, rows_out, R0 + 32 * w, t & 63);
        if ((t & 63) == 0) dstb[w] = d;
    }
    load_tile<kA0Tile>(x, rows, cols, R0, C0, tile, t);
    __syncthreads();
    if (q_row != nullptr) {
        const int64_t nb = cols / 32;
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
            const int u = u2 * 256 + t, r = u >> 2, b = u & 3;
            uint32_t q8[8];
            const uint32_t code = quantize_row_block(tile, r, b, q8);
            const int64_t row = R0 + r, c = C0 + 32 * b;
            if (row < rows && c < cols) {
                v4i *dst = reinterpret_cast<v4i *>(q_row + row * cols + c);
                dst[0] = v4i{(int)q8[0], (int)q8[1], (int)q8[2], (int)q8[3]};
                dst[1] = v4i{(int)q8[4], (int)q8[5], (int)q8[6], (int)q8[7]};
                s_row[row * nb + c / 32] = (uint8_t)code;
            }
        }
    }
    axis0_from_tile(tile, stile, q_col, s_col, rows, cols, R0, C0, t, dstb, rows_out);
}

// Zero codes and zero scale codes (the quantization of zero rows) for every
// 32-row block of q_col / s_col that no source block fills: one workgroup per
// destination block; wave 0 decides, all threads write.
__global__ __launch_bounds__(256) void zero_dst_pads_kernel(uint8_t *__restrict__ q_col, uint8_t *__restrict__ s_col,
                                                            int64_t rows, int64_t cols,
                                                            const int32_t *__restrict__ src_off,
                                                            const int32_t *__restrict__ dst_off, int G,
                                                            int64_t rows_out) {
    __shared__ int pad;
    const int t = threadIdx.x;
    const int64_t d0 = (int64_t)blockIdx.x * 32;
    if (t < 64) {
        // first group whose clamped destination range holds d0
        int found = -1;
        int64_t dlo_f = 0, dhi_f = 0, len_f = 0;
        for (int g0 = 0; g0 < G && found < 0; g0 += 64) {
            const int g = g0 + t;
            int64_t dlo = 0, dhi = 0, lo = 0, hi = 0;
            if (g < G) {
                dlo = dst_off[g];
                dhi = dst_off[g + 1];
                dlo = dlo < 0 ? 0 : (dlo > rows_out ? rows_out : dlo);
                dhi = dhi < dlo ? dlo : (dhi > rows_out ? rows_out : dhi);
                lo = src_off[g];
                hi = src_off[g + 1];
                lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
                hi = hi < lo ? lo : (hi > rows ? rows : hi);
            }
            const unsigned long long hit = __ballot(g < G && d0 >= dlo && d0 < dhi);
            if (hit) {
                const int src = __ffsll((long long)hit) - 1;
                found = g0 + src;
                dlo_f = __shfl(dlo, src);
                dhi_f = __shfl(dhi, src);
                len_f = __shfl(hi - lo, src);
                // filled iff the group's source blocks reach this block (and the
                // group is aligned, as dst_block_of requires)
                const int64_t lo_f = __shfl(lo, src);
                if ((lo_f & 31) || (dlo_f & 31)) len_f = 0;
            }
        }
        if (t == 0) pad = !(found >= 0 && d0 - dlo_f < len_f && d0 + 32 <= dhi_f);
    }
    __syncthreads();
    if (!pad) return;
    const int64_t nbo = rows_out / 32;
    for (int64_t i = t; i < cols * 2; i += 256) {
        const int64_t c = i >> 1;
        *reinterpret_cast<v4i *>(q_col + c * rows_out + d0 + 16 * (i & 1)) = v4i{0, 0, 0, 0};
        if ((i & 1) == 0) s_col[c * nbo + blockIdx.x] = 0;
    }
}

// The same pads in the packed layout of the regrouped grid (N = cols, K =
// rows_out, KS k-steps): destination block d (one workgroup each, over the
// KS * 4 blocks of the layout) that no group fills gets zero codes and scale
// code 0 in every column, as its zero rows quantize; blocks past rows_out and
// rows past cols are the layout's padding (zero codes, scale code 127).
__global__ __launch_bounds__(256) void zero_dst_pads_packed_kernel(uint8_t *__restrict__ qp, uint8_t *__restrict__ sp,
                                                                   int64_t rows, int64_t cols,
                                                                   const int32_t *__restrict__ src_off,
                                                                   const int32_t *__restrict__ dst_off, int G,
                                                                   int64_t rows_out, int64_t KS) {
    __shared__ int pad;
    const int t = threadIdx.x;
    const int64_t d = blockIdx.x, d0 = d * 32;
    if (t < 64) {
        int found = -1;
        int64_t dlo_f = 0, dhi_f = 0, len_f = 0;
        for (int g0 = 0; g0 < G && found < 0 && d0 < rows_out; g0 += 64) {
            const int g = g0 + t;
            int64_t dlo = 0, dhi = 0, lo = 0, hi = 0;
            if (g < G) {
                dlo = dst_off[g];
                dhi = dst_off[g + 1];
                dlo = dlo < 0 ? 0 : (dlo > rows_out ? rows_out : dlo);
                dhi = dhi < dlo ? dlo : (dhi > rows_out ? rows_out : dhi);
                lo = src_off[g];
                hi = src_off[g + 1];
                lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
                hi = hi < lo ? lo : (hi > rows ? rows : hi);
            }
            const unsigned long long hit = __ballot(g < G && d0 >= dlo && d0 < dhi);
            if (hit) {
                const int src = __ffsll((long long)hit) - 1;
                found = g0 + src;
                dlo_f = __shfl(dlo, src);
                dhi_f = __shfl(dhi, src);
                len_f = __shfl(hi - lo, src);
                const int64_t lo_f = __shfl(lo, src);
                if ((lo_f & 31) || (dlo_f & 31)) len_f = 0;
            }
        }
        if (t == 0) pad = d0 >= rows_out ? 2 : !(found >= 0 && d0 - dlo_f < len_f && d0 + 32 <= dhi_f);
    }
    __syncthreads();
    const int kind = pad;                      // 0: filled by the walk, 1: pad block, 2: past rows_out
    const int64_t np = (cols + kPanelRows - 1) / kPanelRows, ks = d / 4;
    const int p = (int)(d & 3);
    for (int64_t f = t; f < np * kPanelRows; f += 256) {
        if (kind == 0 && f < cols) continue;
        const int64_t tl = (f / kPanelRows) * KS + ks;
        const int frow = (int)(f % kPanelRows);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<v4i *>(qp + tl * kTileBytes + frow * kKStep + (((2 * p + h) ^ (frow & 7)) << 4)) =
                v4i{0, 0, 0, 0};
        sp[tl * kScaleStepBytes + (frow >> 4) * 64 + (frow & 15) + 16 * p] =
            (uint8_t)(kind == 1 && f < cols ? 0u : 127u);
    }
}

// ---------------------------------------------------------------- weights -> packed
// Axis-1 quantization of weights [batch][N][K] written straight into the
// GEMM's packed layout (and, if q/scales are given, the canonical grid too):
// one workgroup per (k-step, panel) tile of 256 rows x 128 columns.  Eight
// lanes share a row, lane l owning its 16-element output chunk l % 8 (half a
// 32-block; the block max is completed across the lane pair with one DPP
// swap).  A wave loads its row-groups (8 rows x 256 B each) into registers
// up front, then converts them, so its packed stores are 8 consecutive tile
// rows = one contiguous 1 KB and its canonical stores whole 128-byte row
// segments.  The tile's scale bytes are transposed through LDS into the
// per-lane packed order.  Rows past N and blocks past K/32 hold element 0 and
// scale 127, as repack writes them.
__device__ __forceinline__ int64_t xcd_contiguous_tile(int64_t wg, int64_t nwg) {
    const int64_t q = nwg / 8, r = nwg % 8, x = wg % 8;
    return x * q + (x < r ? x : r) + wg / 8;
}

// waves per workgroup of the packed quantizer (one 256-row tile per
// workgroup; each wave holds 256 / (8 x waves) row-groups).  Measured on
// MI355X, eight against four: the 144-weight sync 5.10 -> 5.00 ms (32 per
// launch) and 6.31 -> 6.11 ms (one per launch), the MLP gate_up weight
// 53.8 -> 52.5 us.
constexpr int kPackedWaves = 8;

// One 256-row x 128-column tile (tile tidx of a [batch][N][K] weight) into the
// packed layout, and into the canonical grid when qc is given.  NT: the code
// stores are nontemporal.  Measured on MI355X over the 144 Qwen3-8B linears,
// 16 per launch: plain 5.37 ms, nontemporal stores 5.16 ms, nontemporal loads
// and stores 5.62 ms, nontemporal loads 5.94 ms; launches that read less than
// the Infinity Cache's size keep plain stores.
template <bool NT>
__device__ __forceinline__ void quantize_packed_tile(const uint16_t *__restrict__ w, uint8_t *__restrict__ qc,
                                                     uint8_t *__restrict__ sc, uint8_t *__restrict__ qp,
                                                     uint32_t *__restrict__ sp, int64_t N, int64_t K,
                                                     int64_t KS, int64_t NP, int64_t tidx,
                                                     uint32_t *codes) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t ks = tidx % KS, panel = (tidx / KS) % NP, b = tidx / (KS * NP);
    const int64_t tile_lin = (b * NP + panel) * KS + ks;
    const int64_t KB = K / 32;
    const int c = lane & 7, blk = c >> 1;
    const int64_t kb = ks * 4 + blk;
    const int64_t k = ks * kKStep + 16 * c;
    constexpr int IT = kPanelRows / (8 * kPackedWaves);        // row-groups per wave

    v4i dl[IT], dh[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int r = (it * kPackedWaves + wv) * 8 + (lane >> 3);
        const int64_t n = panel * kPanelRows + r;
        dl[it] = dh[it] = v4i{0, 0, 0, 0};
        if (n < N && k < K) {
            const v4i *src = reinterpret_cast<const v4i *>(w + (b * N + n) * K + k);
            dl[it] = src[0];
            dh[it] = src[1];
        }
    }

    uint8_t *code_bytes = reinterpret_cast<uint8_t *>(codes);
    uint8_t *qtile = qp + tile_lin * kTileBytes;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int r = (it * kPackedWaves + wv) * 8 + (lane >> 3);
        const uint32_t d[8] = {(uint32_t)dl[it].x, (uint32_t)dl[it].y, (uint32_t)dl[it].z, (uint32_t)dl[it].w,
                               (uint32_t)dh[it].x, (uint32_t)dh[it].y, (uint32_t)dh[it].z, (uint32_t)dh[it].w};
        uint32_t m = max_mag(d, 8);
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadSwap1, 0xF, 0xF, false));
        uint32_t code = scale_code_from_amax_bits(m);
        const int64_t n = panel * kPanelRows + r;
        const bool valid = n < N && kb < KB;
        v4i out;
        if (!valid) {
            code = 127u;
            out = v4i{0, 0, 0, 0};
        } else if (code == 255u) {
            out = v4i{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
        } else {
            const float inv = inv_scale_from_code(code);
            const v2i o0 = convert8(d, inv), o1 = convert8(d + 4, inv);
            out = v4i{o0.x, o0.y, o1.x, o1.y};
        }
        if (qp) {                          // uniform: a job without the packed layout skips it
            v4i *pdst = reinterpret_cast<v4i *>(qtile + r * 128 + ((c ^ (int)swz((uint32_t)r)) << 4));
            if constexpr (NT) __builtin_nontemporal_store(out, pdst);
            else *pdst = out;
        }
        if (qc && valid) {
            v4i *cdst = reinterpret_cast<v4i *>(qc + (b * N + n) * K + k);
            if constexpr (NT) __builtin_nontemporal_store(out, cdst);
            else *cdst = out;
            if ((c & 1) == 0) sc[(b * N + n) * KB + kb] = (uint8_t)code;
        }
        if ((c & 1) == 0) code_bytes[r * 4 + blk] = (uint8_t)code;
    }
    __syncthreads();
    // output word t: rows 16 (t/16) + 4 (t%4) .. +3 of block 4ks + (t/4)%4
    if (sp && t < kPanelRows) {
        const int row0 = 16 * (t >> 4) + 4 * (t & 3), j = (t >> 2) & 3;
        uint32_t o = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) o |= (uint32_t)code_bytes[(row0 + i) * 4 + j] << (8 * i);
        sp[tile_lin * (kScaleStepBytes / 4) + t] = o;
    }
}

// One weight per launch, tiles numbered XCD-contiguously.
template <bool NT>
__global__ __launch_bounds__(kPackedWaves * 64) void quantize_packed_kernel(const uint16_t *__restrict__ w,
                                                              uint8_t *__restrict__ qc,
                                                              uint8_t *__restrict__ sc,
                                                              uint8_t *__restrict__ qp,
                                                              uint32_t *__restrict__ sp, int64_t N,
                                                              int64_t K, int64_t KS, int64_t NP) {
    __shared__ uint32_t codes[kPanelRows];     // [row][block] bytes
    quantize_packed_tile<NT>(w, qc, sc, qp, sp, N, K, KS, NP, xcd_contiguous_tile(blockIdx.x, gridDim.x),
                             codes);
}

// A list of weights in one launch: the workgroups are numbered over the
// concatenated tile lists (XCD-contiguously), and each finds its weight from
// the running tile totals.  The weight number is uniform over the workgroup,
// so its fields come from the kernel-argument segment by scalar loads.  (The
// 2 KB argument table costs about 2 us per launch against the one-weight
// kernel's 72 bytes, measured over 144 launches in a graph, so single weights
// take the kernel above.)
template <bool NT>
__global__ __launch_bounds__(kPackedWaves * 64) void quantize_packed_many_kernel(PackedJobs jobs) {
    __shared__ uint32_t codes[kPanelRows];     // [row][block] bytes
    const int64_t tidx = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    int j = 0;
#pragma unroll
    for (int i = 0; i < kPackedJobsMax - 1; ++i)
        if (i < jobs.count - 1 && tidx >= jobs.tile_end[i]) j = i + 1;
    const int64_t N = jobs.N[j], K = jobs.K[j], start = j ? jobs.tile_end[j - 1] : 0;
    quantize_packed_tile<NT>(jobs.w[j], jobs.qc[j], jobs.sc[j], jobs.qp[j], jobs.sp[j], N, K,
                             (K + kKStep - 1) / kKStep, (N + kPanelRows - 1) / kPanelRows, tidx - start,
                             codes);
}

// axis 0 over a tile walk (cols % 8 == 0); batch matrices x[batch][rows][cols]
template <bool NT>
__global__ __launch_bounds__(256) void quantize_axis0_walk_kernel(const uint16_t *__restrict__ x,
                                                                  uint8_t *__restrict__ q,
                                                                  uint8_t *__restrict__ scales, int64_t rows,
                                                                  int64_t cols, int64_t ntiles) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kA0Tile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kA0Tile * 4];
    const int t = threadIdx.x;
    int64_t idx = blockIdx.x;
    if (idx >= ntiles) return;
    int64_t b, R0, C0;
    tile_origin_of(idx, rows, cols, b, R0, C0);
    v4i v[kA0Loads];
    load_tile_regs<NT>(x + b * rows * cols, rows, cols, R0, C0, t, v);
    for (; idx < ntiles; idx += gridDim.x) {
        store_tile_regs(tile, t, v);
        __syncthreads();
        const int64_t nxt = idx + gridDim.x;
        int64_t b2 = b, R2 = R0, C2 = C0;
        if (nxt < ntiles) {
            tile_origin_of(nxt, rows, cols, b2, R2, C2);
            load_tile_regs<NT>(x + b2 * rows * cols, rows, cols, R2, C2, t, v);
        }
        axis0_from_tile(tile, stile, q + b * rows * cols, scales + b * cols * (rows / 32), rows, cols, R0, C0, t);
        __syncthreads();          // every thread's stores have read the tile
        b = b2;
        R0 = R2;
        C0 = C2;
    }
}

// both axes over a tile walk (cols % 8 == 0).  GROUPED: the axis-0 grid is
// regrouped as quantize_dual_grouped_kernel does (each tile's destination
// blocks found at the top of its iteration; q_row may be null).  Looking the
// next tile's up beside its loads instead (double-buffered) measured no
// faster on the MoE learner's tensors.
template <bool NT, bool GROUPED = false, bool ROW_PACKED = false, bool COL_PACKED = false>
__global__ __launch_bounds__(256) void quantize_dual_walk_kernel(const uint16_t *__restrict__ x,
                                                                 uint8_t *__restrict__ q_row,
                                                                 uint8_t *__restrict__ s_row,
                                                                 uint8_t *__restrict__ q_col,
                                                                 uint8_t *__restrict__ s_col, int64_t rows,
                                                                 int64_t cols, int64_t ntiles,
                                                                 const int32_t *__restrict__ src_off = nullptr,
                                                                 const int32_t *__restrict__ dst_off = nullptr,
                                                                 int G = 0, int64_t rows_out = 0) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kA0Tile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kA0Tile * 4];
    __shared__ int dstb[4];
    const int t = threadIdx.x;
    int64_t idx = blockIdx.x;
    if (idx >= ntiles) return;
    // ROW_PACKED: the axis-1 grid goes straight into the packed layout (N =
    // rows, K = cols), the walk running over the rows of whole panels so that
    // a half panel past the matrix writes its padding (zero codes, scale code
    // 127) and nothing of axis 0
    const int64_t rows_walk = ROW_PACKED ? (rows + kPanelRows - 1) / kPanelRows * kPanelRows : rows;
    const int64_t KS1 = (cols + kKStep - 1) / kKStep;
    int64_t b_unused, R0, C0;
    tile_origin_of(idx, rows_walk, cols, b_unused, R0, C0);
    v4i v[kA0Loads];
    load_tile_regs<NT>(x, rows, cols, R0, C0, t, v);
    const int64_t nb = cols / 32;
    for (; idx < ntiles; idx += gridDim.x) {
        if constexpr (GROUPED) {
            // wave w finds the destination of the tile's source block w (read
            // after the barriers below; the previous tile's readers ended at
            // the barrier closing the last iteration)
            const int w = t >> 6;
            const int d = dst_block_of(src_off, dst_off, G, rows, rows_out, R0 + 32 * w, t & 63);
            if ((t & 63) == 0) dstb[w] = d;
        }
        store_tile_regs(tile, t, v);
        __syncthreads();
        const int64_t nxt = idx + gridDim.x;
        int64_t R2 = R0, C2 = C0;
        if (nxt < ntiles) {
            tile_origin_of(nxt, rows_walk, cols, b_unused, R2, C2);
            load_tile_regs<NT>(x, rows, cols, R2, C2, t, v);
        }
        if constexpr (ROW_PACKED) {
            // rows R0 .. R0+127 are half (R0 / 128) % 2 of panel R0 / 256 at
            // k-step C0 / 128 (as quantize_dual_packed_kernel)
            const int64_t tl = (R0 / kPanelRows) * KS1 + C0 / kKStep;
            const int half = (int)((R0 / kA0Tile) & 1);
            uint8_t *qt = q_row + tl * kTileBytes + half * (kA0Tile * kKStep);
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                const int u = u2 * 256 + t, r = u >> 2, bb = u & 3;
                uint32_t q8[8];
                uint32_t code = quantize_row_block(tile, r, bb, q8);
                if (R0 + r >= rows || C0 + 32 * bb >= cols) code = 127u;    // padding (its codes are zero)
                const int sw = r & 7;
                *reinterpret_cast<v4i *>(qt + r * kKStep + (((2 * bb) ^ sw) << 4)) =
                    v4i{(int)q8[0], (int)q8[1], (int)q8[2], (int)q8[3]};
                *reinterpret_cast<v4i *>(qt + r * kKStep + (((2 * bb + 1) ^ sw) << 4)) =
                    v4i{(int)q8[4], (int)q8[5], (int)q8[6], (int)q8[7]};
                const int rp = half * kA0Tile + r;
                s_row[tl * kScaleStepBytes + (rp >> 4) * 64 + (rp & 15) + 16 * bb] = (uint8_t)code;
            }
        } else if (!GROUPED || q_row != nullptr) {
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                const int u = u2 * 256 + t, r = u >> 2, bb = u & 3;
                uint32_t q8[8];
                const uint32_t code = quantize_row_block(tile, r, bb, q8);
                const int64_t row = R0 + r, c = C0 + 32 * bb;
                if (row < rows && c < cols) {
                    v4i *dst = reinterpret_cast<v4i *>(q_row + row * cols + c);
                    dst[0] = v4i{(int)q8[0], (int)q8[1], (int)q8[2], (int)q8[3]};
                    dst[1] = v4i{(int)q8[4], (int)q8[5], (int)q8[6], (int)q8[7]};
                    s_row[row * nb + c / 32] = (uint8_t)code;
                }
            }
        }
        if (!ROW_PACKED || R0 < rows) {       // (uniform over the workgroup)
            // COL_PACKED: the regrouped grid in the packed layout (N = cols,
            // K = rows_out)
            if constexpr (COL_PACKED)
                axis0_from_tile_packed(tile, stile, q_col, s_col, cols, C0, t, dstb, (rows_out + kKStep - 1) / kKStep);
            else if constexpr (GROUPED)
                axis0_from_tile(tile, stile, q_col, s_col, rows, cols, R0, C0, t, dstb, rows_out);
            else
                axis0_from_tile(tile, stile, q_col, s_col, rows, cols, R0, C0, t);
        }
        __syncthreads();
        R0 = R2;
        C0 = C2;
    }
}

// Axis 0 straight into the packed layout of the transposed grid: x[batch]
// [rows][cols] quantized along rows (as the axis-0 kernel) and written as
// mxfp8_repack lays out q[batch][cols][rows] (N' = cols, K' = rows).  A
// 128x128 tile is one k-step (its 128 rows) of one half-panel (its 128
// columns), so the tile list covers two halves of every panel, and a half
// beyond cols writes the panel's padding (zero codes, scale code 127), as do
// the blocks beyond rows.  Walks tiles as quantize_axis0_walk_kernel does.
__device__ __forceinline__ void packed_t_tile_origin(int64_t idx, int64_t KS, int64_t NP2, int64_t &b,
                                                     int64_t &R0, int64_t &C0) {
    const int64_t per = KS * NP2, t = idx % per;
    b = idx / per;
    R0 = (t / NP2) * kA0Tile;
    C0 = (t % NP2) * kA0Tile;
}

template <bool NT>
__global__ __launch_bounds__(256) void quantize_axis0_packed_kernel(const uint16_t *__restrict__ x,
                                                                    uint8_t *__restrict__ qp,
                                                                    uint32_t *__restrict__ sp, int64_t rows,
                                                                    int64_t cols, int64_t ntiles) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kA0Tile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kA0Tile * 4];
    const int t = threadIdx.x;
    const int64_t KS = (rows + kKStep - 1) / kKStep, NP = (cols + kPanelRows - 1) / kPanelRows;
    int64_t idx = blockIdx.x;
    if (idx >= ntiles) return;
    int64_t b, R0, C0;
    packed_t_tile_origin(idx, KS, 2 * NP, b, R0, C0);
    v4i v[kA0Loads];
    load_tile_regs<NT>(x + b * rows * cols, rows, cols, R0, C0, t, v);
    for (; idx < ntiles; idx += gridDim.x) {
        store_tile_regs(tile, t, v);
        __syncthreads();
        const int64_t nxt = idx + gridDim.x;
        int64_t b2 = b, R2 = R0, C2 = C0;
        if (nxt < ntiles) {
            packed_t_tile_origin(nxt, KS, 2 * NP, b2, R2, C2);
            load_tile_regs<NT>(x + b2 * rows * cols, rows, cols, R2, C2, t, v);
        }
        axis0_stage_tile(tile, stile, t);
        // codes: output row o = C0 + col is row o % 256 of panel o / 256 in
        // k-step R0 / 128; chunk j (input rows R0 + 16j ..) at slot j ^ (o % 8).
        // Loads beyond rows or cols were zero, so those codes are zero.
        const int64_t ks = R0 / kKStep, h = (C0 / kA0Tile) & 1;
        const int64_t tile_lin = (b * NP + C0 / kPanelRows) * KS + ks;
        uint8_t *qt = qp + tile_lin * kTileBytes + h * (kA0Tile * kKStep);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = i * 32 + (t >> 3), j = t & 7;
            *reinterpret_cast<v4i *>(qt + col * kKStep + ((j ^ (col & 7)) << 4)) =
                *reinterpret_cast<const v4i *>(tile + col * kA0OutPitch + 16 * j);
        }
        // scales: words h*128 .. h*128+127 of the k-step's 1 KB scale tile; word
        // w holds rows 16(w/16) + 4(w%4) .. +3 (of the panel) of block (w/4) % 4
        if (t < kA0Tile) {
            const int jb = (t >> 2) & 3;
            uint32_t o = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int lc = 16 * (t >> 4) + 4 * (t & 3) + i;
                const uint32_t code =
                    (C0 + lc < cols && R0 + 32 * jb < rows) ? (uint32_t)stile[lc * 4 + jb] : 127u;
                o |= code << (8 * i);
            }
            sp[tile_lin * (kScaleStepBytes / 4) + h * kA0Tile + t] = o;
        }
        __syncthreads();          // every thread's stores have read the staged tile
        b = b2;
        R0 = R2;
        C0 = C2;
    }
}

// Both axes straight into the packed layouts: one BF16 read of x[rows][cols]
// gives what mxfp8_repack writes for the axis-1 grid (q[rows][cols]; N = rows,
// K = cols) and for the axis-0 grid (q[cols][rows]; N' = cols, K' = rows).  A
// 128x128 tile is half a panel by one k-step of both layouts; the walk covers
// every half panel of both (rows and cols rounded up to 256) of every matrix
// of the batch, so tiles and blocks beyond a matrix write the layouts'
// padding (zero codes, scale code 127).  The axis-1 codes are stored first
// (each thread's two blocks of a row as four 16-byte chunks at their swizzled
// slots), then the tile is staged for axis 0 exactly as
// quantize_axis0_packed_kernel stores it.
template <bool NT>
__global__ __launch_bounds__(256) void quantize_dual_packed_kernel(const uint16_t *__restrict__ x,
                                                                   uint8_t *__restrict__ qr, uint8_t *__restrict__ sr,
                                                                   uint8_t *__restrict__ qc, uint32_t *__restrict__ sc,
                                                                   int64_t rows, int64_t cols, int64_t ntiles) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kA0Tile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t stile[kA0Tile * 4];
    const int t = threadIdx.x;
    const int64_t KS1 = (cols + kKStep - 1) / kKStep, KS0 = (rows + kKStep - 1) / kKStep;
    const int64_t NPr = (rows + kPanelRows - 1) / kPanelRows, NPc = (cols + kPanelRows - 1) / kPanelRows;
    const int64_t CT = 2 * NPc;                                          // column half-panels
    const int64_t TPM = 2 * NPr * CT;                                    // tiles per matrix
    int64_t idx = blockIdx.x;
    if (idx >= ntiles) return;
    // tile idx: matrix idx / TPM, its rows R0.. and columns C0..
    auto tile_of = [&](int64_t i, int64_t &b, int64_t &R, int64_t &C) {
        b = i / TPM;
        const int64_t r = i % TPM;
        R = (r / CT) * kA0Tile;
        C = (r % CT) * kA0Tile;
    };
    int64_t b0, R0, C0;
    tile_of(idx, b0, R0, C0);
    v4i v[kA0Loads];
    load_tile_regs<NT>(x + b0 * rows * cols, rows, cols, R0, C0, t, v);
    for (; idx < ntiles; idx += gridDim.x) {
        store_tile_regs(tile, t, v);
        __syncthreads();
        const int64_t nxt = idx + gridDim.x;
        int64_t b2 = b0, R2 = R0, C2 = C0;
        if (nxt < ntiles) {
            tile_of(nxt, b2, R2, C2);
            load_tile_regs<NT>(x + b2 * rows * cols, rows, cols, R2, C2, t, v);
        }
        if (C0 < KS1 * kKStep) {
            // axis 1: rows R0 .. R0+127 are half (R0 / 128) % 2 of panel R0 / 256
            // at k-step C0 / 128
            const int64_t tl = (b0 * NPr + R0 / kPanelRows) * KS1 + C0 / kKStep;
            const int half = (int)((R0 / kA0Tile) & 1);
            uint8_t *qt = qr + tl * kTileBytes + half * (kA0Tile * kKStep);
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                const int u = u2 * 256 + t, r = u >> 2, bb = u & 3;
                uint32_t q8[8];
                uint32_t code = quantize_row_block(tile, r, bb, q8);
                if (R0 + r >= rows || C0 + 32 * bb >= cols) code = 127u;    // padding (its codes are zero)
                const int sw = r & 7;
                *reinterpret_cast<v4i *>(qt + r * kKStep + (((2 * bb) ^ sw) << 4)) =
                    v4i{(int)q8[0], (int)q8[1], (int)q8[2], (int)q8[3]};
                *reinterpret_cast<v4i *>(qt + r * kKStep + (((2 * bb + 1) ^ sw) << 4)) =
                    v4i{(int)q8[4], (int)q8[5], (int)q8[6], (int)q8[7]};
                const int rp = half * kA0Tile + r;                        // row in the panel
                sr[tl * kScaleStepBytes + (rp >> 4) * 64 + (rp & 15) + 16 * bb] = (uint8_t)code;
            }
        }
        if (R0 < KS0 * kKStep) {
            axis0_stage_tile(tile, stile, t);
            // axis 0: output row o = C0 + col is row o % 256 of panel o / 256 in
            // k-step R0 / 128 (as quantize_axis0_packed_kernel)
            const int64_t ks = R0 / kKStep, h = (C0 / kA0Tile) & 1;
            const int64_t tile_lin = (b0 * NPc + C0 / kPanelRows) * KS0 + ks;
            uint8_t *qt = qc + tile_lin * kTileBytes + h * (kA0Tile * kKStep);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = i * 32 + (t >> 3), j = t & 7;
                *reinterpret_cast<v4i *>(qt + col * kKStep + ((j ^ (col & 7)) << 4)) =
                    *reinterpret_cast<const v4i *>(tile + col * kA0OutPitch + 16 * j);
            }
            if (t < kA0Tile) {
                const int jb = (t >> 2) & 3;
                uint32_t o = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lc = 16 * (t >> 4) + 4 * (t & 3) + i;
                    const uint32_t code =
                        (C0 + lc < cols && R0 + 32 * jb < rows) ? (uint32_t)stile[lc * 4 + jb] : 127u;
                    o |= code << (8 * i);
                }
                sc[tile_lin * (kScaleStepBytes / 4) + h * kA0Tile + t] = o;
            }
        }
        __syncthreads();          // every thread's stores have read the tile
        b0 = b2;
        R0 = R2;
        C0 = C2;
    }
}

// Workgroups of a tile walk: as many per CU as can be resident at once, at
// most one per tile.  The LDS tile would allow four per CU, but the walks'
// 130-145 registers per lane leave room for three 256-thread workgroups; with
// four per CU in the grid the fourth waits for a whole walk to end (measured
// on MI355X, three instead of four: axis 0 on 24576x4096 4.82 -> 5.33 TB/s,
// 16384x16384 5.24 -> 5.44; both axes level or up to 8% faster).  The count
// comes from the runtime's occupancy query for each kernel, once.
template <auto Kernel>
static int64_t walk_grid(int64_t ntiles) {
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(Kernel), 256, 0) !=
                hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    const int64_t cap = (int64_t)device_cu_count() * per_cu;
    return ntiles < cap ? ntiles : cap;
}

hipError_t launch_quantize(const uint16_t *x, int64_t rows, int64_t cols, int axis, uint8_t *q,
                           uint8_t *scales, hipStream_t stream) {
    if (axis == 1) {
        const int64_t nblocks = rows * (cols / 32);
        const int64_t nsteps = (nblocks + 63) / 64;
        // a fixed number of waves per CU, each walking several steps
        const bool nt = rows * cols * 2 >= kQuantNontemporalBytes;
        int64_t grid = (nsteps + 3) / 4;
        const int64_t cap = (int64_t)device_cu_count() * ((nt ? kQuantWavesPerCuLarge : kQuantWavesPerCu) / 4);
        if (grid > cap) grid = cap;
        if (grid < 1) grid = 1;
        if (nt)
            hipLaunchKernelGGL(quantize_axis1_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x, q,
                               scales, nblocks);
        else
            hipLaunchKernelGGL(quantize_axis1_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, x, q,
                               scales, nblocks);
    } else {
        return launch_quantize_axis0_batched(x, 1, rows, cols, q, scales, stream);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_many(const QuantJobs &jobs, hipStream_t stream) {
    const int64_t nsteps = jobs.step_end[jobs.count - 1];
    bool packed = false;
    for (int i = 0; i < jobs.count; ++i) packed = packed || jobs.packed[i];
    int64_t grid = (nsteps + 3) / 4;
    // workgroups of 4 waves resident per CU: 8 (<= 64 registers), 6 with packed jobs (<= 80)
    const int64_t cap = (int64_t)device_cu_count() * (packed ? 6 : kQuantWavesPerCu / 4);
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    if (packed) hipLaunchKernelGGL(quantize_axis1_many_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, jobs);
    else hipLaunchKernelGGL(quantize_axis1_many_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, jobs);
    return hipGetLastError();
}

hipError_t launch_quantize_axis0_batched(const uint16_t *x, int64_t batch, int64_t rows,
                                         int64_t cols, uint8_t *q, uint8_t *scales,
                                         hipStream_t stream) {
    const int64_t tiles = ((rows + kA0Tile - 1) / kA0Tile) * ((cols + kA0Tile - 1) / kA0Tile);
    if (cols % 8 == 0) {
        const int64_t grid = walk_grid<quantize_axis0_walk_kernel<true>>(batch * tiles);
        hipLaunchKernelGGL(quantize_axis0_walk_kernel<true>, dim3((unsigned)grid), dim3(256),
                           0, stream, x, q, scales, rows, cols, batch * tiles);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(quantize_axis0_kernel, dim3((unsigned)(batch * tiles)), dim3(256), 0, stream,
                       x, q, scales, rows, cols);
    return hipGetLastError();
}

hipError_t launch_quantize_axis0_packed(const uint16_t *x, int64_t batch, int64_t rows, int64_t cols,
                                        uint8_t *q_packed, uint8_t *s_packed, hipStream_t stream) {
    const int64_t ntiles = batch * packed_ksteps(rows) * 2 * packed_panels(cols);
    uint32_t *sp = reinterpret_cast<uint32_t *>(s_packed);
    if (batch * rows * cols * 2 >= kQuantNontemporalBytes) {
        const int64_t grid = walk_grid<quantize_axis0_packed_kernel<true>>(ntiles);
        hipLaunchKernelGGL(quantize_axis0_packed_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                           q_packed, sp, rows, cols, ntiles);
    } else {
        const int64_t grid = walk_grid<quantize_axis0_packed_kernel<false>>(ntiles);
        hipLaunchKernelGGL(quantize_axis0_packed_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                           q_packed, sp, rows, cols, ntiles);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_gather(const uint16_t *x, int64_t rows_in, int64_t cols,
                                  const int64_t *idx, int64_t rows_out, uint8_t *q,
                                  uint8_t *scales, hipStream_t stream) {
    const int64_t bpr = cols / 32;
    const int64_t nblocks = rows_out * bpr;
    const int64_t nsteps = (nblocks + 63) / 64;
    int64_t grid = (nsteps + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * (kGatherWavesPerCu / 4);
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(quantize_gather_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x,
                       rows_in, bpr, idx, q, scales, nblocks);
    return hipGetLastError();
}

hipError_t launch_quantize_gather_packed(const uint16_t *x, int64_t rows_in, int64_t cols, const int64_t *idx,
                                         int64_t rows_out, uint8_t *q_packed, uint8_t *s_packed, hipStream_t stream) {
    const int64_t nsteps = packed_panels(rows_out) * 16 * packed_ksteps(cols);
    // six 4-wave workgroups per CU, as the list quantizer's packed variant
    int64_t grid = (nsteps + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 6;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(quantize_gather_packed_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, rows_in, cols,
                       idx, rows_out, q_packed, s_packed, nsteps);
    return hipGetLastError();
}

hipError_t launch_quantize_dual(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_row,
                                uint8_t *s_row, uint8_t *q_col, uint8_t *s_col, hipStream_t stream) {
    const int64_t tiles = ((rows + kA0Tile - 1) / kA0Tile) * ((cols + kA0Tile - 1) / kA0Tile);
    if (cols % 8 == 0) {
        if (rows * cols * 2 >= kQuantNontemporalBytes) {
            const int64_t grid = walk_grid<quantize_dual_walk_kernel<true>>(tiles);
            hipLaunchKernelGGL(quantize_dual_walk_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                               q_row, s_row, q_col, s_col, rows, cols, tiles);
        } else {
            const int64_t grid = walk_grid<quantize_dual_walk_kernel<false>>(tiles);
            hipLaunchKernelGGL(quantize_dual_walk_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                               q_row, s_row, q_col, s_col, rows, cols, tiles);
        }
        return hipGetLastError();
    }
    hipLaunchKernelGGL(quantize_dual_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, x, q_row,
                       s_row, q_col, s_col, rows, cols);
    return hipGetLastError();
}

hipError_t launch_quantize_dual_packed(const uint16_t *x, int64_t batch, int64_t rows, int64_t cols,
                                       uint8_t *qr_packed, uint8_t *sr_packed, uint8_t *qc_packed,
                                       uint8_t *sc_packed, hipStream_t stream) {
    const int64_t tiles = batch * 2 * packed_panels(rows) * 2 * packed_panels(cols);
    uint32_t *sc = reinterpret_cast<uint32_t *>(sc_packed);
    if (batch * rows * cols * 2 >= kQuantNontemporalBytes) {
        const int64_t grid = walk_grid<quantize_dual_packed_kernel<true>>(tiles);
        hipLaunchKernelGGL(quantize_dual_packed_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                           qr_packed, sr_packed, qc_packed, sc, rows, cols, tiles);
    } else {
        const int64_t grid = walk_grid<quantize_dual_packed_kernel<false>>(tiles);
        hipLaunchKernelGGL(quantize_dual_packed_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                           qr_packed, sr_packed, qc_packed, sc, rows, cols, tiles);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_dual_grouped(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_row,
                                        uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                                        const int32_t *src_off, const int32_t *dst_off, int64_t G,
                                        int64_t rows_out, hipStream_t stream) {
    hipLaunchKernelGGL(zero_dst_pads_kernel, dim3((unsigned)(rows_out / 32)), dim3(256), 0, stream, q_col,
                       s_col, rows, cols, src_off, dst_off, (int)G, rows_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t tiles = ((rows + kA0Tile - 1) / kA0Tile) * ((cols + kA0Tile - 1) / kA0Tile);
    if (cols % 8 == 0) {
        // nontemporal loads from inputs of the Infinity Cache's size, as the
        // plain dual walk (measured: the MoE learner's dY 65536x2048 162 -> 144
        // us, X 122 -> 117 us)
        if (rows * cols * 2 >= kQuantNontemporalBytes) {
            const int64_t grid = walk_grid<quantize_dual_walk_kernel<true, true>>(tiles);
            hipLaunchKernelGGL((quantize_dual_walk_kernel<true, true>), dim3((unsigned)grid), dim3(256), 0, stream,
                               x, q_row, s_row, q_col, s_col, rows, cols, tiles, src_off, dst_off, (int)G,
                               rows_out);
            return hipGetLastError();
        }
        const int64_t grid = walk_grid<quantize_dual_walk_kernel<false, true>>(tiles);
        hipLaunchKernelGGL((quantize_dual_walk_kernel<false, true>), dim3((unsigned)grid), dim3(256), 0, stream, x,
                           q_row, s_row, q_col, s_col, rows, cols, tiles, src_off, dst_off, (int)G, rows_out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(quantize_dual_grouped_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, x, q_row,
                       s_row, q_col, s_col, rows, cols, src_off, dst_off, (int)G, rows_out);
    return hipGetLastError();
}

template <bool ROWP, bool COLP>
static hipError_t launch_dual_grouped_packed_walk(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qr,
                                                  uint8_t *sr, uint8_t *qc, uint8_t *sc, const int32_t *src_off,
                                                  const int32_t *dst_off, int64_t G, int64_t rows_out,
                                                  int64_t tiles, hipStream_t stream) {
    if (rows * cols * 2 >= kQuantNontemporalBytes) {
        const int64_t grid = walk_grid<quantize_dual_walk_kernel<true, true, ROWP, COLP>>(tiles);
        hipLaunchKernelGGL((quantize_dual_walk_kernel<true, true, ROWP, COLP>), dim3((unsigned)grid), dim3(256), 0,
                           stream, x, qr, sr, qc, sc, rows, cols, tiles, src_off, dst_off, (int)G, rows_out);
    } else {
        const int64_t grid = walk_grid<quantize_dual_walk_kernel<false, true, ROWP, COLP>>(tiles);
        hipLaunchKernelGGL((quantize_dual_walk_kernel<false, true, ROWP, COLP>), dim3((unsigned)grid), dim3(256), 0,
                           stream, x, qr, sr, qc, sc, rows, cols, tiles, src_off, dst_off, (int)G, rows_out);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_dual_grouped_packed(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qr_packed,
                                               uint8_t *sr_packed, uint8_t *qc, uint8_t *sc, bool col_packed,
                                               const int32_t *src_off, const int32_t *dst_off, int64_t G,
                                               int64_t rows_out, hipStream_t stream) {
    // the regrouped grid's pad blocks (and, packed, the layout's padding)
    // first: the walk's stores, later on the stream, win wherever a
    // malformed table overlaps them
    const int64_t KS = packed_ksteps(rows_out);
    if (col_packed)
        hipLaunchKernelGGL(zero_dst_pads_packed_kernel, dim3((unsigned)(KS * 4)), dim3(256), 0, stream, qc, sc, rows,
                           cols, src_off, dst_off, (int)G, rows_out, KS);
    else
        hipLaunchKernelGGL(zero_dst_pads_kernel, dim3((unsigned)(rows_out / 32)), dim3(256), 0, stream, qc, sc, rows,
                           cols, src_off, dst_off, (int)G, rows_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // with the row grid packed, the walk runs over whole panels of rows
    // (cols % 32 == 0, so rows are 16-byte aligned for the walk's loads)
    const int64_t tc = (cols + kA0Tile - 1) / kA0Tile;
    const int64_t tiles_r = 2 * packed_panels(rows) * tc, tiles = ((rows + kA0Tile - 1) / kA0Tile) * tc;
    if (qr_packed != nullptr)
        return col_packed ? launch_dual_grouped_packed_walk<true, true>(x, rows, cols, qr_packed, sr_packed, qc, sc,
                                                                       src_off, dst_off, G, rows_out, tiles_r, stream)
                          : launch_dual_grouped_packed_walk<true, false>(x, rows, cols, qr_packed, sr_packed, qc, sc,
                                                                        src_off, dst_off, G, rows_out, tiles_r, stream);
    return col_packed ? launch_dual_grouped_packed_walk<false, true>(x, rows, cols, nullptr, nullptr, qc, sc, src_off,
                                                                    dst_off, G, rows_out, tiles, stream)
                      : launch_dual_grouped_packed_walk<false, false>(x, rows, cols, nullptr, nullptr, qc, sc, src_off,
                                                                     dst_off, G, rows_out, tiles, stream);
}

hipError_t launch_quantize_packed_jobs(const PackedJobs &jobs, hipStream_t stream) {
    const int64_t tiles = jobs.tile_end[jobs.count - 1];
    int64_t bytes = 0;
    for (int i = 0; i < jobs.count; ++i) {
        const int64_t start = i ? jobs.tile_end[i - 1] : 0;
        bytes += (jobs.tile_end[i] - start) * kTileBytes * 2;     // BF16 read, counted in whole tiles
    }
    if (bytes >= kQuantNontemporalBytes)
        hipLaunchKernelGGL(quantize_packed_many_kernel<true>, dim3((unsigned)tiles), dim3(kPackedWaves * 64), 0,
                           stream, jobs);
    else
        hipLaunchKernelGGL(quantize_packed_many_kernel<false>, dim3((unsigned)tiles), dim3(kPackedWaves * 64), 0,
                           stream, jobs);
    return hipGetLastError();
}

hipError_t launch_quantize_packed(const uint16_t *w, int64_t batch, int64_t N, int64_t K,
                                  uint8_t *q, uint8_t *scales, uint8_t *q_packed,
                                  uint8_t *s_packed, hipStream_t stream) {
    const int64_t NP = packed_panels(N), KS = packed_ksteps(K), tiles = batch * NP * KS;
    uint32_t *sp = reinterpret_cast<uint32_t *>(s_packed);
    if (tiles * kTileBytes * 2 >= kQuantNontemporalBytes)
        hipLaunchKernelGGL(quantize_packed_kernel<true>, dim3((unsigned)tiles), dim3(kPackedWaves * 64), 0,
                           stream, w, q, scales, q_packed, sp, N, K, KS, NP);
    else
        hipLaunchKernelGGL(quantize_packed_kernel<false>, dim3((unsigned)tiles), dim3(kPackedWaves * 64), 0,
                           stream, w, q, scales, q_packed, sp, N, K, KS, NP);
    return hipGetLastError();
}

}  // namespace mx
