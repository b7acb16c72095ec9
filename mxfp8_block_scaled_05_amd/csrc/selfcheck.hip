// Post-sync self-check kernels (gfx950).
//
// The page's post-sync self-check ("End-to-End MXFP8 RL on Blackwell" (verl
// blog), section "Correctness: how it fails", run-time check C3) runs one
// quantized layer through the serving kernel on random input and compares it
// with a high-precision GEMM on the dequantized synchronized weights: a
// healthy layer is a few percent off (the activation quantization), a stale
// derived layout is off by order 1.  Here:
//   - the serving path is the library's own quantize + MXFP8 GEMM against
//     the packed storage the sampler's graphs read (launched by the API);
//   - ref_gemm_kernel computes the reference from the canonical synchronized
//     grid, dequantizing each weight on the fly, in fp32;
//   - the relative Frobenius error ||Y - Y_ref|| / ||Y_ref|| is reduced in
//     fp64 in a fixed order (deterministic), NaN if either output is not
//     finite.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

constexpr int kRefTile = 64;
constexpr int kRefK = 32;

// Y_ref[M][N] = X[M][K] * W'[N][K]^T, W' = decode(q) * 2^(s - 127), fp32.
// 64 x 64 output tile per workgroup, 4 x 4 outputs per thread.
__global__ __launch_bounds__(256) void ref_gemm_kernel(const uint16_t *__restrict__ x,
                                                       const uint8_t *__restrict__ wq,
                                                       const uint8_t *__restrict__ ws,
                                                       float *__restrict__ y, int64_t M, int64_t N,
                                                       int64_t K) {
    __shared__ float xa[kRefK][kRefTile + 1];
    __shared__ float wb[kRefK][kRefTile + 1];
    const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * kRefTile, n0 = (int64_t)blockIdx.x * kRefTile;
    const int64_t KB = K / 32;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += kRefK) {
#pragma unroll
        for (int i = 0; i < kRefTile * kRefK / 256; ++i) {
            const int e = i * 256 + t, r = e / kRefK, kk = e % kRefK;
            const int64_t m = m0 + r, n = n0 + r;
            xa[kk][r] = m < M ? bits_to_float((uint32_t)x[m * K + k0 + kk] << 16) : 0.f;
            float wv = 0.f;
            if (n < N) {
                const float v = __builtin_amdgcn_cvt_f32_fp8((int)wq[n * K + k0 + kk], 0);
                wv = ldexpf(v, (int)ws[n * KB + k0 / 32] - 127);
            }
            wb[kk][r] = wv;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kRefK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xa[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = wb[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n < N) y[m * N + n] = acc[i][j];
        }
    }
}

constexpr int kErrBlocks = 256;

// Per-workgroup partial sums of (y - r)^2 and r^2 (fp64), grid-stride over
// a fixed grid, tree-reduced in LDS: the same inputs give the same bits.
__global__ __launch_bounds__(256) void sq_err_partials_kernel(const float *__restrict__ y,
                                                              const float *__restrict__ r,
                                                              int64_t n, double *__restrict__ part) {
    __shared__ double sa[256], sb[256];
    double a = 0.0, b = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const double d = (double)y[i] - (double)r[i];
        a += d * d;
        b += (double)r[i] * (double)r[i];
    }
    sa[threadIdx.x] = a;
    sb[threadIdx.x] = b;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            sa[threadIdx.x] += sa[threadIdx.x + s];
            sb[threadIdx.x] += sb[threadIdx.x + s];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = sa[0];
        part[2 * blockIdx.x + 1] = sb[0];
    }
}

// out[0] = sqrt(sum a / sum b) (NaN if a sum is not finite or b is 0),
// out[1] = sum a, out[2] = sum b.
__global__ __launch_bounds__(256) void sq_err_final_kernel(const double *__restrict__ part, int nparts,
                                                           double *__restrict__ out) {
    __shared__ double sa[256], sb[256];
    double a = 0.0, b = 0.0;
    for (int i = threadIdx.x; i < nparts; i += 256) {
        a += part[2 * i];
        b += part[2 * i + 1];
    }
    sa[threadIdx.x] = a;
    sb[threadIdx.x] = b;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            sa[threadIdx.x] += sa[threadIdx.x + s];
            sb[threadIdx.x] += sb[threadIdx.x + s];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double num = sa[0], den = sb[0];
        const bool ok = __builtin_isfinite(num) && __builtin_isfinite(den) && den > 0.0;
        out[0] = ok ? __builtin_sqrt(num / den) : __builtin_nan("");
        out[1] = num;
        out[2] = den;
    }
}

SelfcheckWorkspace selfcheck_workspace(int64_t M, int64_t N, int64_t K) {
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    SelfcheckWorkspace w;
    w.xq = 0;
    w.xs = up(M * K);
    w.y = w.xs + up(M * (K / 32));
    w.yref = w.y + up(M * N * 4);
    w.part = w.yref + up(M * N * 4);
    w.total = w.part + up(kErrBlocks * 2 * 8);
    return w;
}

hipError_t launch_selfcheck_ref(const uint16_t *x, int64_t M, int64_t N, int64_t K,
                                const uint8_t *wq, const uint8_t *ws, float *yref,
                                hipStream_t stream) {
    dim3 grid((unsigned)((N + kRefTile - 1) / kRefTile), (unsigned)((M + kRefTile - 1) / kRefTile));
    hipLaunchKernelGGL(ref_gemm_kernel, grid, dim3(256), 0, stream, x, wq, ws, yref, M, N, K);
    return hipGetLastError();
}

hipError_t launch_selfcheck_error(const float *y, const float *yref, int64_t n, double *part,
                                  double *out, hipStream_t stream) {
    hipLaunchKernelGGL(sq_err_partials_kernel, dim3(kErrBlocks), dim3(256), 0, stream, y, yref, n,
                       part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sq_err_final_kernel, dim3(1), dim3(256), 0, stream, part, kErrBlocks, out);
    return hipGetLastError();
}

}  // namespace mx
