// Canonical MXFP8 weights -> the GEMM's packed kernel layout (gfx950).
//
// The page's sampler rebuilds its kernel-specific weight and scale layouts
// from the canonical tensors after every weight synchronization ("End-to-End
// MXFP8 RL on Blackwell" (verl blog), section "The pipeline", sampler
// paragraph: swizzled scales, shuffled experts, repacked weights); this is
// that rebuild for the gfx950 GEMM.  Pure byte permutation, HBM-bound at
// 2.0625 algorithmic bytes per element.  The layout is specified in
// include/mxfp8.h (mxfp8_repack):
//   elements: [batch][panel of 256 rows][k-step of 128][256 rows][128 B], the
//             16-byte chunk c of row r stored at slot c ^ f(r % 16) -- exactly
//             the GEMM's LDS image of a B tile, so the GEMM copies it linearly.
//   scales  : [batch][panel][k-step][16 atoms of 16 rows][64 lanes] bytes --
//             one byte per MFMA lane per atom, 1 KB per panel and k-step, so
//             the GEMM copies a tile's scales of one step as one block.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

// One workgroup per (k-step, panel, batch) tile of 32 KB.  Eight consecutive
// lanes move one 128-byte row, so loads and stores are whole rows.
__global__ __launch_bounds__(256) void repack_q_kernel(const uint8_t *__restrict__ q,
                                                       uint8_t *__restrict__ qp, int64_t N,
                                                       int64_t K) {
    const int64_t ks = blockIdx.x, panel = blockIdx.y, b = blockIdx.z;
    const int64_t KS = gridDim.x, NP = gridDim.y;
    uint8_t *dst = qp + ((b * NP + panel) * KS + ks) * kTileBytes;
    const uint8_t *src = q + b * N * K;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int ci = it * 256 + threadIdx.x;
        const int r = ci >> 3, c = ci & 7;
        const int64_t n = panel * kPanelRows + r;
        const int64_t k = ks * kKStep + c * 16;
        v4i v = v4i{0, 0, 0, 0};
        if (n < N && k < K) v = *reinterpret_cast<const v4i *>(src + n * K + k);
        *reinterpret_cast<v4i *>(dst + r * 128 + ((c ^ (int)swz(r)) * 16)) = v;
    }
}

// One thread per output dword: bytes (panel, k-step, atom, lanes l..l+3) are
// the scales of rows 256*panel + 16*atom + (l % 16) .. +3, block 4*kstep +
// l/16 (four consecutive rows, one block); padding holds 127.
__global__ __launch_bounds__(256) void repack_s_kernel(const uint8_t *__restrict__ s,
                                                       uint32_t *__restrict__ sp, int64_t batch,
                                                       int64_t N, int64_t K, int64_t NP,
                                                       int64_t KS) {
    const int64_t total = batch * NP * KS * (kScaleStepBytes / 4);
    const int64_t nb = K / 32;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t lane0 = (i * 4) & 63;
        const int64_t atom = (i >> 4) & 15;
        const int64_t ks = (i >> 8) % KS;
        const int64_t panel = (i >> 8) / KS % NP;
        const int64_t b = (i >> 8) / (KS * NP);
        const int64_t blk = 4 * ks + (lane0 >> 4);
        const int64_t row0 = panel * kPanelRows + atom * 16 + (lane0 & 15);
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = row0 + q;
            uint32_t v = 127u;
            if (n < N && blk < nb) v = s[(b * N + n) * nb + blk];
            word |= v << (8 * q);
        }
        sp[i] = word;
    }
}

hipError_t launch_repack(const uint8_t *q, const uint8_t *scales, int64_t batch, int64_t N,
                         int64_t K, uint8_t *q_packed, uint8_t *s_packed, hipStream_t stream) {
    const int64_t NP = packed_panels(N), KS = packed_ksteps(K);
    dim3 grid((unsigned)KS, (unsigned)NP, (unsigned)batch);
    hipLaunchKernelGGL(repack_q_kernel, grid, dim3(256), 0, stream, q, q_packed, N, K);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = batch * NP * KS * (kScaleStepBytes / 4);
    int64_t g = (total + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(repack_s_kernel, dim3((unsigned)g), dim3(256), 0, stream, scales,
                       reinterpret_cast<uint32_t *>(s_packed), batch, N, K, NP, KS);
    return hipGetLastError();
}

}  // namespace mx
