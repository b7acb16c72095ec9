// Canonical MXFP8 weights -> the GEMM's packed kernel layout (gfx950).
//
// The page's sampler rebuilds its kernel-specific weight and scale layouts
// from the canonical tensors after every weight synchronization ("End-to-End
// MXFP8 RL on Blackwell" (verl blog), section "The pipeline", sampler
// paragraph: the serving kernels read rearranged copies of weights and
// scales, regenerated at every update); this is that rebuild for the gfx950 GEMM.  Pure byte permutation, HBM-bound at
// 2.0625 algorithmic bytes per element.  The layout is specified in
// include/mxfp8.h (mxfp8_repack):
//   elements: [batch][panel of 256 rows][k-step of 128][256 rows][128 B], the
//             16-byte chunk c of row r stored at slot c ^ (r % 8) -- exactly
//             the GEMM's LDS image of a B tile, so the GEMM copies it linearly.
//   scales  : [batch][panel][k-step][16 atoms of 16 rows][64 lanes] bytes --
//             one byte per MFMA lane per atom, 1 KB per panel and k-step, so
//             the GEMM copies a tile's scales of one step as one block.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

// Workgroup index -> tile index such that each XCD (workgroups are dealt to
// the eight XCDs round-robin) gets a contiguous range of tiles: all k-steps of
// a panel then run under one L2, which serves the panel's scale rows to every
// k-step after the first.
__device__ __forceinline__ int64_t xcd_contiguous(int64_t wg, int64_t nwg) {
    const int64_t q = nwg / 8, r = nwg % 8, x = wg % 8;
    return x * q + (x < r ? x : r) + wg / 8;
}

// One workgroup per (k-step, panel, batch) tile.
//  - elements: 32 KB; eight consecutive lanes move one 128-byte row, so loads
//    and stores are whole rows.
//  - scales: the tile's 1 KB.  Thread t loads the four scale bytes (blocks
//    4ks .. 4ks+3) of panel row t as one word, the words meet in LDS, and
//    thread t then gathers its output word: rows 16*(t/16) + 4*(t%4) .. +3 of
//    block 4ks + (t/4)%4, i.e. bytes (atom t/16, lanes 4*(t%16) .. +3).
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t *__restrict__ q,
                                                     const uint8_t *__restrict__ s,
                                                     uint8_t *__restrict__ qp,
                                                     uint32_t *__restrict__ sp, int64_t N,
                                                     int64_t K, int64_t KS, int64_t NP) {
    __shared__ uint32_t rows_s[kPanelRows];
    const int t = threadIdx.x;
    const int64_t tile = xcd_contiguous(blockIdx.x, gridDim.x);
    const int64_t ks = tile % KS, panel = (tile / KS) % NP, b = tile / (KS * NP);
    const int64_t tile_lin = (b * NP + panel) * KS + ks;

    // scale word of row t: blocks 4ks .. 4ks+3, padding 127
    const int64_t nb = K / 32, n = panel * kPanelRows + t, blk0 = 4 * ks;
    uint32_t word = 0x7F7F7F7Fu;
    if (n < N) {
        const uint8_t *srow = s + (b * N + n) * nb;
        if ((nb & 3) == 0) {
            word = *reinterpret_cast<const uint32_t *>(srow + blk0);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (blk0 + j < nb)
                    word = (word & ~(0xFFu << (8 * j))) | ((uint32_t)srow[blk0 + j] << (8 * j));
        }
    }
    rows_s[t] = word;

    uint8_t *dst = qp + tile_lin * kTileBytes;
    const uint8_t *src = q + b * N * K;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int ci = it * 256 + t;
        const int r = ci >> 3, c = ci & 7;
        const int64_t nr = panel * kPanelRows + r;
        const int64_t k = ks * kKStep + c * 16;
        v4i v = v4i{0, 0, 0, 0};
        if (nr < N && k < K) v = *reinterpret_cast<const v4i *>(src + nr * K + k);
        *reinterpret_cast<v4i *>(dst + r * 128 + ((c ^ (int)swz(r)) * 16)) = v;
    }

    __syncthreads();
    const uint8_t *bytes = reinterpret_cast<const uint8_t *>(rows_s);
    const int row0 = 16 * (t >> 4) + 4 * (t & 3), j = (t >> 2) & 3;
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) out |= (uint32_t)bytes[(row0 + i) * 4 + j] << (8 * i);
    sp[tile_lin * (kScaleStepBytes / 4) + t] = out;
}

hipError_t launch_repack(const uint8_t *q, const uint8_t *scales, int64_t batch, int64_t N,
                         int64_t K, uint8_t *q_packed, uint8_t *s_packed, hipStream_t stream) {
    const int64_t NP = packed_panels(N), KS = packed_ksteps(K);
    const int64_t tiles = batch * NP * KS;
    hipLaunchKernelGGL(repack_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, q, scales,
                       q_packed, reinterpret_cast<uint32_t *>(s_packed), N, K, KS, NP);
    return hipGetLastError();
}

}  // namespace mx
