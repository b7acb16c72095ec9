// MXFP8 dequantizer kernels for gfx950:  out = decode(q) * 2^(code - 127).
//
// The reference side of the page's post-sync self-check is a high-precision
// GEMM on dequantized synchronized weights ("End-to-End MXFP8 RL on
// Blackwell" (verl blog), section "Correctness: how it fails", "Post-sync
// self-check").  HBM-bound: 1 + 1/32 bytes in, 4 (fp32) or 2 (bf16) out per
// element.  E4M3 -> fp32 uses the hardware OCP conversion (exact), the scale
// is applied with ldexp (exact, including fp32 subnormal results).
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void decode4(uint32_t w, int e, float *o) {
    v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    o[0] = __builtin_amdgcn_ldexpf(a.x, e);
    o[1] = __builtin_amdgcn_ldexpf(a.y, e);
    o[2] = __builtin_amdgcn_ldexpf(b.x, e);
    o[3] = __builtin_amdgcn_ldexpf(b.y, e);
}

// decode 16 elements sharing one scale code
__device__ __forceinline__ void decode16(v4i w, uint32_t code, float *o) {
    const int e = (int)code - 127;
    decode4((uint32_t)w.x, e, o);
    decode4((uint32_t)w.y, e, o + 4);
    decode4((uint32_t)w.z, e, o + 8);
    decode4((uint32_t)w.w, e, o + 12);
    if (code == 255u) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = __builtin_nanf("");
    }
}

__device__ __forceinline__ void store16(void *out, int64_t idx, const float *v, bool bf16) {
    if (bf16) {
        uint32_t p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = bf16x2_rne(v[2 * i], v[2 * i + 1]);
        v4i *dst = reinterpret_cast<v4i *>(static_cast<uint16_t *>(out) + idx);
        dst[0] = v4i{(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
        dst[1] = v4i{(int)p[4], (int)p[5], (int)p[6], (int)p[7]};
    } else {
        v4f *dst = reinterpret_cast<v4f *>(static_cast<float *>(out) + idx);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = v4f{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    }
}

// axis 1: flat, 16 elements per lane (blocks never straddle rows).
__global__ __launch_bounds__(256) void dequantize_axis1_kernel(const uint8_t *__restrict__ q,
                                                               const uint8_t *__restrict__ s,
                                                               void *__restrict__ out, int64_t nchunks,
                                                               bool bf16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks; i += stride) {
        const v4i w = *reinterpret_cast<const v4i *>(q + i * 16);
        const uint32_t code = s[i >> 1];
        float v[16];
        decode16(w, code, v);
        store16(out, i * 16, v, bf16);
    }
}

// axis 0: q[cols][rows] -> out[rows][cols] through a 64x64 LDS transpose.
__global__ __launch_bounds__(256) void dequantize_axis0_kernel(const uint8_t *__restrict__ q,
                                                               const uint8_t *__restrict__ s,
                                                               void *__restrict__ out, int64_t rows,
                                                               int64_t cols, bool bf16) {
    __shared__ float tile[64][65];
    const int t = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int64_t r0 = (int64_t)blockIdx.y * 64;
    {   // load: thread -> (column c0 + t/4, rows r0 + 16*(t%4) .. +15)
        const int cc = t >> 2, seg = t & 3;
        const int64_t c = c0 + cc, r = r0 + seg * 16;
        float v[16];
        if (c < cols && r < rows) {
            const v4i w = *reinterpret_cast<const v4i *>(q + c * rows + r);
            decode16(w, s[c * (rows / 32) + r / 32], v);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tile[cc][seg * 16 + i] = v[i];
    }
    __syncthreads();
    {   // store: thread -> (row r0 + t/4, columns c0 + 16*(t%4) .. +15)
        const int rr = t >> 2, seg = t & 3;
        const int64_t r = r0 + rr, c = c0 + seg * 16;
        if (r >= rows || c >= cols) return;
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = tile[seg * 16 + i][rr];
        if (c + 16 <= cols && ((cols & (bf16 ? 7 : 3)) == 0)) {
            store16(out, r * cols + c, v, bf16);
        } else {
            for (int i = 0; i < 16 && c + i < cols; ++i) {
                if (bf16) static_cast<uint16_t *>(out)[r * cols + c + i] = (uint16_t)f32_to_bf16_rne(v[i]);
                else static_cast<float *>(out)[r * cols + c + i] = v[i];
            }
        }
    }
}

hipError_t launch_dequantize(const uint8_t *q, const uint8_t *scales, int64_t rows, int64_t cols,
                             int axis, void *out, bool out_bf16, hipStream_t stream) {
    if (axis == 1) {
        const int64_t nchunks = rows * cols / 16;
        int64_t grid = (nchunks + 255) / 256;
        const int64_t cap = (int64_t)device_cu_count() * 32;
        if (grid > cap) grid = cap;
        if (grid < 1) grid = 1;
        hipLaunchKernelGGL(dequantize_axis1_kernel, dim3((unsigned)grid), dim3(256), 0, stream, q,
                           scales, out, nchunks, out_bf16);
    } else {
        dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
        hipLaunchKernelGGL(dequantize_axis0_kernel, grid, dim3(256), 0, stream, q, scales, out,
                           rows, cols, out_bf16);
    }
    return hipGetLastError();
}

}  // namespace mx
