// Host-side launchers of the gfx950 MXFP8 kernels (internal to the library;
// the public C ABI is include/mxfp8.h).  Every launcher assumes its
// arguments were validated by the API layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Compute units of the current device (cached per device).
int device_cu_count();

// Dense GEMM tiling: big_cols tile columns of 256x256 tiles over the leading
// columns, then small_cols tile columns of 256x128 tiles (either may be 0).
struct DenseTiling {
    int big_cols, small_cols;
};
DenseTiling dense_tiling(int64_t M, int64_t N, int cus);

// Split-K plan of a dense GEMM: K slices of split_steps k-steps, fp32
// partials of splits * M * N floats (splits == 1: no split).
struct SplitPlan {
    int splits, split_steps;
    int64_t workspace_bytes;
};
SplitPlan splitk_plan(int64_t M, int64_t N, int64_t K, int cus);
// partial tiles into `workspace`, then C = their sum (slice order)
// mxfp8_gemm_accurate: BF16 MFMA on exactly converted operands
hipError_t launch_gemm_accurate(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                const uint8_t *b_s, bool b_packed, int64_t M, int64_t N, int64_t K, void *c,
                                bool c_bf16, hipStream_t stream);
// device address and size of the static split-K scratch on the current device
hipError_t splitk_scratch(void **ptr, size_t *bytes);
hipError_t launch_gemm_splitk(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q, const uint8_t *b_s,
                              bool b_packed, int64_t M, int64_t N, int64_t K, void *c, bool c_bf16,
                              const SplitPlan &plan, float *workspace, hipStream_t stream);

hipError_t launch_quantize(const uint16_t *x, int64_t rows, int64_t cols, int axis, uint8_t *q,
                           uint8_t *scales, hipStream_t stream);

// x[batch][rows][cols] -> q[batch][cols][rows], scales[batch][cols][rows/32]
hipError_t launch_quantize_axis0_batched(const uint16_t *x, int64_t batch, int64_t rows,
                                         int64_t cols, uint8_t *q, uint8_t *scales,
                                         hipStream_t stream);

// axis-1 quantize of rows x[idx[i]] (zero rows for indices outside [0, rows_in))
hipError_t launch_quantize_gather(const uint16_t *x, int64_t rows_in, int64_t cols,
                                  const int64_t *idx, int64_t rows_out, uint8_t *q,
                                  uint8_t *scales, hipStream_t stream);

hipError_t launch_quantize_dual(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_row,
                                uint8_t *s_row, uint8_t *q_col, uint8_t *s_col, hipStream_t stream);
hipError_t launch_quantize_gather_packed(const uint16_t *x, int64_t rows_in, int64_t cols, const int64_t *idx,
                                         int64_t rows_out, uint8_t *q_packed, uint8_t *s_packed, hipStream_t stream);
hipError_t launch_quantize_dual_grouped_packed(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qr_packed,
                                               uint8_t *sr_packed, uint8_t *qc, uint8_t *sc, bool col_packed,
                                               const int32_t *src_off, const int32_t *dst_off, int64_t G,
                                               int64_t rows_out, hipStream_t stream);
hipError_t launch_grouped_gemm_wgrad_packed(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                            const uint8_t *b_s, const int32_t *offsets, int64_t G, int64_t T,
                                            int64_t M, int64_t N, void *c, bool c_bf16, hipStream_t stream);
hipError_t launch_quantize_dual_packed(const uint16_t *x, int64_t batch, int64_t rows, int64_t cols,
                                       uint8_t *qr_packed, uint8_t *sr_packed, uint8_t *qc_packed,
                                       uint8_t *sc_packed, hipStream_t stream);

// axis 1 (q_row / s_row may be null) and axis 0 regrouped by token offsets
// into q_col[cols][rows_out], s_col[cols][rows_out/32], pads zeroed
hipError_t launch_quantize_dual_grouped(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_row,
                                        uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                                        const int32_t *src_off, const int32_t *dst_off, int64_t G,
                                        int64_t rows_out, hipStream_t stream);

// x[batch][rows][cols] along axis 0 into the packed layout of the transposed
// grid (what repack writes for q[batch][cols][rows]); rows % 32 == 0,
// cols % 8 == 0
hipError_t launch_quantize_axis0_packed(const uint16_t *x, int64_t batch, int64_t rows, int64_t cols,
                                        uint8_t *q_packed, uint8_t *s_packed, hipStream_t stream);

// Several tensors quantized along axis 1 in one launch.  Tensor i has
// nblocks[i] = rows * cols / 32 blocks and ceil(nblocks[i] / 64) wave-steps,
// which are steps step_end[i-1] .. step_end[i]-1 of the launch.
constexpr int kQuantJobsMax = 8;
struct QuantJobs {
    const uint16_t *x[kQuantJobsMax];
    uint8_t *q[kQuantJobsMax];
    uint8_t *s[kQuantJobsMax];
    int64_t nblocks[kQuantJobsMax];
    int64_t step_end[kQuantJobsMax];
    // packed[i]: q/s of job i are the packed layout of its grid; its steps are
    // (16-row atom, k-step) pairs over ceil(rows / 256) * 16 atoms
    int64_t rows[kQuantJobsMax];
    int64_t cols[kQuantJobsMax];
    int32_t packed[kQuantJobsMax];
    int count;
};
hipError_t launch_quantize_many(const QuantJobs &jobs, hipStream_t stream);

// A list of weights quantized into the packed layout in one launch.  Weight i
// is BF16 [batch_i][N[i]][K[i]]; its tiles are tile_end[i-1] .. tile_end[i]-1
// of the launch (tile_end[i] - tile_end[i-1] = batch_i * panels * k-steps).
constexpr int kPackedJobsMax = 32;
struct PackedJobs {
    const uint16_t *w[kPackedJobsMax];
    uint8_t *qc[kPackedJobsMax];      // canonical q, or null
    uint8_t *sc[kPackedJobsMax];      // canonical scales, or null
    uint8_t *qp[kPackedJobsMax];
    uint32_t *sp[kPackedJobsMax];
    int64_t N[kPackedJobsMax];
    int64_t K[kPackedJobsMax];
    int64_t tile_end[kPackedJobsMax];
    int count;
};
hipError_t launch_quantize_packed_jobs(const PackedJobs &jobs, hipStream_t stream);

// q / scales may be null (packed output only)
hipError_t launch_quantize_packed(const uint16_t *w, int64_t batch, int64_t N, int64_t K,
                                  uint8_t *q, uint8_t *scales, uint8_t *q_packed,
                                  uint8_t *s_packed, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t *q, const uint8_t *scales, int64_t rows, int64_t cols,
                             int axis, void *out, bool out_bf16, hipStream_t stream);

hipError_t launch_repack(const uint8_t *q, const uint8_t *scales, int64_t batch, int64_t N,
                         int64_t K, uint8_t *q_packed, uint8_t *s_packed, hipStream_t stream);

// the tiles launch_gemm_packed takes: gemm_ws_kernel's 256x128 or 128x128
// tiles, or launch_gemm's tilings
enum class PackedTiling { kWs, kWsHalf, kDense };
PackedTiling packed_tiling(int64_t M, int64_t N, bool c_bf16, int cus);
hipError_t launch_gemm_packed(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q, const uint8_t *b_s,
                              int64_t M, int64_t N, int64_t K, void *c, bool c_bf16, hipStream_t stream);
hipError_t launch_gemm_packed_splitk(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                     const uint8_t *b_s, int64_t M, int64_t N, int64_t K, void *c,
                                     bool c_bf16, const SplitPlan &sp, float *workspace, hipStream_t stream);
hipError_t launch_grouped_gemm_packed(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                      const uint8_t *b_s, const int32_t *offsets, int64_t G, int64_t M_total,
                                      int64_t N, int64_t K, void *c, bool c_bf16, hipStream_t stream);
hipError_t launch_gemm(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                       const uint8_t *b_s, bool b_packed, int64_t M, int64_t N, int64_t K, void *c,
                       bool c_bf16, hipStream_t stream);

hipError_t launch_grouped_gemm(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                               const uint8_t *b_s, const int32_t *offsets, int64_t G,
                               int64_t M_total, int64_t N, int64_t K, void *c, bool c_bf16,
                               hipStream_t stream);

// Self-check workspace: byte offsets of its parts (256-byte aligned) and the
// total size, for a probe of M rows against weights [N][K].
struct SelfcheckWorkspace {
    int64_t xq, xs, y, yref, part, total;
};
SelfcheckWorkspace selfcheck_workspace(int64_t M, int64_t N, int64_t K);

// Reference Y_ref = X * dequant(W)^T in fp32 (X bf16 [M][K], W canonical [N][K]).
hipError_t launch_selfcheck_ref(const uint16_t *x, int64_t M, int64_t N, int64_t K,
                                const uint8_t *wq, const uint8_t *ws, float *yref,
                                hipStream_t stream);

// out[0] = ||y - yref|| / ||yref|| (NaN if not finite), out[1..2] the sums.
hipError_t launch_selfcheck_error(const float *y, const float *yref, int64_t n, double *part,
                                  double *out, hipStream_t stream);

// C[g] = A[:, o_g:o_g+1] B[:, o_g:o_g+1]^T, A [M][T], B [N][T] canonical (row stride T)
hipError_t launch_grouped_gemm_wgrad(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                     const uint8_t *b_s, const int32_t *offsets, int64_t G,
                                     int64_t T, int64_t M, int64_t N, void *c, bool c_bf16,
                                     hipStream_t stream);

// Packed weight layout geometry (see mxfp8_repack in include/mxfp8.h).
constexpr int64_t kPanelRows = 256;   // rows per packed panel
constexpr int64_t kKStep = 128;       // K bytes per packed k-step (one MFMA K)
constexpr int64_t kTileBytes = kPanelRows * kKStep;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t packed_panels(int64_t N) { return ceil_div(N, kPanelRows); }
inline int64_t packed_ksteps(int64_t K) { return ceil_div(K, kKStep); }
inline int64_t packed_q_bytes(int64_t batch, int64_t N, int64_t K) {
    return batch * packed_panels(N) * packed_ksteps(K) * kTileBytes;
}
// scales: [batch][panel][k-step][16 atoms of 16 rows][64 lanes] bytes
constexpr int64_t kScaleStepBytes = 16 * 64;
inline int64_t packed_s_bytes(int64_t batch, int64_t N, int64_t K) {
    return batch * packed_panels(N) * packed_ksteps(K) * kScaleStepBytes;
}

}  // namespace mx
