// C ABI of the gfx950 MXFP8 library: argument validation and kernel dispatch.
// The contract of every entry point is documented in include/mxfp8.h.
#include "mxfp8.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "mx_launch.hpp"

namespace mx {

static thread_local int g_last_hip_error = 0;

namespace {
struct DeviceInfo {
    bool valid = false;
    bool gfx950 = false;
    int cus = 0;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

const DeviceInfo *current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
        g_dev[dev].cus = prop.multiProcessorCount;
        g_dev[dev].gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_dev[dev].valid = true;
    });
    return g_dev[dev].valid ? &g_dev[dev] : nullptr;
}
}  // namespace

int device_cu_count() {
    const DeviceInfo *d = current_device();
    return (d && d->cus > 0) ? d->cus : 256;
}

// 1 if the current device is gfx950, 0 if not, -1 if it cannot be queried
int device_arch_ok() {
    const DeviceInfo *d = current_device();
    if (!d) return -1;
    return d->gfx950 ? 1 : 0;
}

}  // namespace mx

using namespace mx;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;     // any single dimension
constexpr int64_t kMaxK = (int64_t)1 << 22;       // 256 rows x K must stay < 2^31 B
constexpr int64_t kMaxSelfcheckRows = 4096;       // probe rows of a self-check

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The integer a caller passed for an enum parameter.  C callers may pass any
// int; reading such a value through the enum type is undefined in C++ (the
// host UBSan build flags it), so enum arguments are validated on their bytes.
template <class E>
int raw(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
    int v = 0;
    memcpy(&v, &e, sizeof v);
    return v;
}

mxfp8_status check_device() {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXFP8_ERR_HIP;
    }
    const int arch = device_arch_ok();
    if (arch < 0) return MXFP8_ERR_HIP;
    return arch ? MXFP8_OK : MXFP8_ERR_UNSUPPORTED;
}

mxfp8_status finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MXFP8_ERR_HIP;
    }
    return MXFP8_OK;
}

// the axis-0 and dual quantizers run one workgroup per 128x128 tile on a
// one-dimensional grid
bool tile128_ok(int64_t rows, int64_t cols) {
    return ((rows + 127) / 128) * ((cols + 127) / 128) <= 0x7FFFFFFF;
}

// repack runs one workgroup of 256 threads per (matrix, panel, k-step) tile on
// a one-dimensional grid: keep the thread count below 2^32
bool repack_tiles_ok(int64_t batch, int64_t rows, int64_t cols) {
    return batch * packed_panels(rows) * packed_ksteps(cols) < ((int64_t)1 << 24);
}

}  // namespace

extern "C" {

const char *mxfp8_version(void) { return "0.1.0"; }

int mxfp8_last_hip_error(void) { return g_last_hip_error; }

const char *mxfp8_status_string(mxfp8_status s) {
    switch (s) {
        case MXFP8_OK: return "MXFP8_OK";
        case MXFP8_ERR_NULL: return "MXFP8_ERR_NULL: a required pointer is NULL";
        case MXFP8_ERR_SHAPE: return "MXFP8_ERR_SHAPE: invalid or unsupported size";
        case MXFP8_ERR_AXIS: return "MXFP8_ERR_AXIS: axis must be 0 or 1";
        case MXFP8_ERR_DTYPE: return "MXFP8_ERR_DTYPE: unknown dtype or layout";
        case MXFP8_ERR_ALIGN: return "MXFP8_ERR_ALIGN: pointer not 16-byte aligned";
        case MXFP8_ERR_HIP: return "MXFP8_ERR_HIP: HIP launch or query failed";
        case MXFP8_ERR_UNSUPPORTED: return "MXFP8_ERR_UNSUPPORTED: device is not gfx950";
    }
    return "MXFP8: unknown status";
}

mxfp8_status mxfp8_quantize(const void *x_bf16, int64_t rows, int64_t cols, int axis, uint8_t *q,
                            uint8_t *scales, hipStream_t stream) {
    if (!x_bf16 || !q || !scales) return MXFP8_ERR_NULL;
    if (axis != 0 && axis != 1) return MXFP8_ERR_AXIS;
    if (rows <= 0 || cols <= 0 || rows >= kMaxDim || cols >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (axis == 1 && cols % 32) return MXFP8_ERR_SHAPE;
    if (axis == 0 && (rows % 32 || !tile128_ok(rows, cols))) return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q) || !aligned16(scales)) return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize(static_cast<const uint16_t *>(x_bf16), rows, cols, axis, q,
                                  scales, stream));
}

mxfp8_status mxfp8_quantize_batched(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols,
                                    int axis, uint8_t *q, uint8_t *scales, hipStream_t stream) {
    if (!x_bf16 || !q || !scales) return MXFP8_ERR_NULL;
    if (axis != 0 && axis != 1) return MXFP8_ERR_AXIS;
    if (batch <= 0 || batch > 65535 || rows <= 0 || cols <= 0 || rows >= kMaxDim || cols >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    if (batch * rows >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (axis == 1 && cols % 32) return MXFP8_ERR_SHAPE;
    if (axis == 0 && (rows % 32 || !tile128_ok(batch * rows, cols))) return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q) || !aligned16(scales)) return MXFP8_ERR_ALIGN;
    if (axis == 0 && (rows * cols) % 16) return MXFP8_ERR_ALIGN;      // every matrix 16-byte aligned
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    if (axis == 1) return finish(launch_quantize(x, batch * rows, cols, 1, q, scales, stream));
    return finish(launch_quantize_axis0_batched(x, batch, rows, cols, q, scales, stream));
}

mxfp8_status mxfp8_quantize_gather(const void *x_bf16, int64_t rows_in, int64_t cols,
                                   const int64_t *d_row_index, int64_t rows_out, uint8_t *q,
                                   uint8_t *scales, hipStream_t stream) {
    if (!x_bf16 || !d_row_index || !q || !scales) return MXFP8_ERR_NULL;
    if (rows_in <= 0 || rows_out <= 0 || cols <= 0 || cols % 32 || rows_in >= kMaxDim ||
        rows_out >= kMaxDim || cols >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q) || ((uintptr_t)d_row_index & 7u)) return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_gather(static_cast<const uint16_t *>(x_bf16), rows_in, cols,
                                         d_row_index, rows_out, q, scales, stream));
}

mxfp8_status mxfp8_quantize_gather_packed(const void *x_bf16, int64_t rows_in, int64_t cols,
                                          const int64_t *d_row_index, int64_t rows_out, uint8_t *q_packed,
                                          uint8_t *s_packed, hipStream_t stream) {
    if (!x_bf16 || !d_row_index || !q_packed || !s_packed) return MXFP8_ERR_NULL;
    if (rows_in <= 0 || rows_out <= 0 || cols <= 0 || cols % 32 || rows_in >= kMaxDim || rows_out >= kMaxDim ||
        cols > kMaxK)
        return MXFP8_ERR_SHAPE;
    // the packed layout within mxfp8_repack's limits; the atom walk's step
    // count within 2^31
    if (!repack_tiles_ok(1, rows_out, cols) || packed_panels(rows_out) * 16 * packed_ksteps(cols) >= ((int64_t)1 << 31))
        return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q_packed) || !aligned16(s_packed) || ((uintptr_t)d_row_index & 7u))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_gather_packed(static_cast<const uint16_t *>(x_bf16), rows_in, cols, d_row_index,
                                                rows_out, q_packed, s_packed, stream));
}

mxfp8_status mxfp8_grouped_gemm_wgrad_packed(const uint8_t *a_q_packed, const uint8_t *a_s_packed,
                                             const uint8_t *b_q_packed, const uint8_t *b_s_packed,
                                             const int32_t *d_group_offsets, int64_t G, int64_t T, int64_t M,
                                             int64_t N, void *c, mxfp8_dtype c_dtype, hipStream_t stream) {
    if (!a_q_packed || !a_s_packed || !b_q_packed || !b_s_packed || !d_group_offsets || !c) return MXFP8_ERR_NULL;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    const bool bf = raw(c_dtype) == MXFP8_BF16;
    if (G < 1 || G > 65535 || T < 32 || T % 32 || T > kMaxK) return MXFP8_ERR_SHAPE;
    if (M <= 0 || N <= 0 || M >= kMaxDim || N >= kMaxDim || N % (bf ? 8 : 4)) return MXFP8_ERR_SHAPE;
    // both packed operands within mxfp8_repack's limits; C's row stores
    // through 32-bit buffer offsets; the unit count within 2^31
    if (!repack_tiles_ok(1, M, T) || !repack_tiles_ok(1, N, T) || (int64_t)128 * N * (bf ? 2 : 4) >= ((int64_t)1 << 31) ||
        G * ((M + 255) / 256) * ((N + 127) / 128) > 0x7FFFFFFF)
        return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q_packed) || !aligned16(a_s_packed) || !aligned16(b_q_packed) || !aligned16(b_s_packed) ||
        !aligned16(c) || ((uintptr_t)d_group_offsets & 3u))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_grouped_gemm_wgrad_packed(a_q_packed, a_s_packed, b_q_packed, b_s_packed, d_group_offsets, G,
                                                   T, M, N, c, bf, stream));
}

mxfp8_status mxfp8_grouped_gemm_wgrad(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                      const uint8_t *b_s, const int32_t *d_group_offsets,
                                      int64_t G, int64_t T, int64_t M, int64_t N, void *c,
                                      mxfp8_dtype c_dtype, hipStream_t stream) {
    if (!a_q || !a_s || !b_q || !b_s || !d_group_offsets || !c) return MXFP8_ERR_NULL;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (G < 1 || G > 65535 || T < 32 || T % 32 || T >= ((int64_t)1 << 23)) return MXFP8_ERR_SHAPE;
    if (M <= 0 || N <= 0 || M >= kMaxDim || N >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (G * ((M + 255) / 256) * ((N + 255) / 256) > 0x7FFFFFFF) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q) || !aligned16(b_s) || !aligned16(c) ||
        ((uintptr_t)d_group_offsets & 3u))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_grouped_gemm_wgrad(a_q, a_s, b_q, b_s, d_group_offsets, G, T, M, N, c,
                                            raw(c_dtype) == MXFP8_BF16, stream));
}

mxfp8_status mxfp8_quantize_dual(const void *x_bf16, int64_t rows, int64_t cols, uint8_t *q_row,
                                 uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                                 hipStream_t stream) {
    if (!x_bf16 || !q_row || !s_row || !q_col || !s_col) return MXFP8_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows >= kMaxDim || cols >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (rows % 32 || cols % 32 || !tile128_ok(rows, cols)) return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q_row) || !aligned16(s_row) || !aligned16(q_col) ||
        !aligned16(s_col))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_dual(static_cast<const uint16_t *>(x_bf16), rows, cols, q_row,
                                       s_row, q_col, s_col, stream));
}

mxfp8_status mxfp8_quantize_dual_packed(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols,
                                        uint8_t *q_row_packed, uint8_t *s_row_packed, uint8_t *q_col_packed,
                                        uint8_t *s_col_packed, hipStream_t stream) {
    if (!x_bf16 || !q_row_packed || !s_row_packed || !q_col_packed || !s_col_packed) return MXFP8_ERR_NULL;
    if (batch <= 0 || batch > 65535 || rows <= 0 || cols <= 0 || rows % 32 || cols % 32) return MXFP8_ERR_SHAPE;
    // both packed layouts within mxfp8_repack's limits, and the tile walk's
    // count (half panels of both, over the batch) within 2^31
    if (rows >= kMaxDim || cols >= kMaxDim || rows > kMaxK || cols > kMaxK || !repack_tiles_ok(batch, rows, cols) ||
        !repack_tiles_ok(batch, cols, rows) ||
        batch * 4 * packed_panels(rows) * packed_panels(cols) >= ((int64_t)1 << 31) ||
        batch * rows * cols >= ((int64_t)1 << 50))
        return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q_row_packed) || !aligned16(s_row_packed) || !aligned16(q_col_packed) ||
        !aligned16(s_col_packed))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_dual_packed(static_cast<const uint16_t *>(x_bf16), batch, rows, cols,
                                              q_row_packed, s_row_packed, q_col_packed, s_col_packed, stream));
}

mxfp8_status mxfp8_quantize_dual_grouped(const void *x_bf16, int64_t rows, int64_t cols, uint8_t *q_row,
                                         uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                                         const int32_t *src_offsets, const int32_t *dst_offsets, int64_t G,
                                         int64_t rows_out, hipStream_t stream) {
    if (!x_bf16 || !q_col || !s_col || !src_offsets || !dst_offsets) return MXFP8_ERR_NULL;
    if ((q_row == nullptr) != (s_row == nullptr)) return MXFP8_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows >= kMaxDim || cols >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (rows % 32 || cols % 32 || !tile128_ok(rows, cols)) return MXFP8_ERR_SHAPE;
    if (G < 1 || G > 65535 || rows_out <= 0 || rows_out % 32 || rows_out >= kMaxDim ||
        rows_out / 32 > 0x7FFFFFFF)
        return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q_col) || (q_row && (!aligned16(q_row) || !aligned16(s_row))) ||
        ((uintptr_t)src_offsets & 3u) || ((uintptr_t)dst_offsets & 3u))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_dual_grouped(static_cast<const uint16_t *>(x_bf16), rows, cols, q_row, s_row,
                                               q_col, s_col, src_offsets, dst_offsets, G, rows_out, stream));
}

mxfp8_status mxfp8_quantize_dual_grouped_packed(const void *x_bf16, int64_t rows, int64_t cols,
                                                uint8_t *q_row_packed, uint8_t *s_row_packed, uint8_t *q_col,
                                                uint8_t *s_col, mxfp8_layout col_layout, const int32_t *src_offsets,
                                                const int32_t *dst_offsets, int64_t G, int64_t rows_out,
                                                hipStream_t stream) {
    if (!x_bf16 || !q_col || !s_col || !src_offsets || !dst_offsets) return MXFP8_ERR_NULL;
    if ((q_row_packed == nullptr) != (s_row_packed == nullptr)) return MXFP8_ERR_NULL;
    if (raw(col_layout) != MXFP8_CANONICAL && raw(col_layout) != MXFP8_PACKED) return MXFP8_ERR_DTYPE;
    const bool col_packed = raw(col_layout) == MXFP8_PACKED;
    if (rows <= 0 || cols <= 0 || rows >= kMaxDim || cols >= kMaxDim || cols > kMaxK) return MXFP8_ERR_SHAPE;
    if (rows % 32 || cols % 32 || !tile128_ok(rows, cols)) return MXFP8_ERR_SHAPE;
    if (G < 1 || G > 65535 || rows_out <= 0 || rows_out % 32 || rows_out >= kMaxDim ||
        rows_out / 32 > 0x7FFFFFFF || (col_packed && rows_out > kMaxK))
        return MXFP8_ERR_SHAPE;
    // the packed layouts within mxfp8_repack's limits; the walk (over whole
    // panels of rows with the row grid) within 2^31 tiles
    if ((col_packed && !repack_tiles_ok(1, cols, rows_out)) || (q_row_packed && !repack_tiles_ok(1, rows, cols)) ||
        2 * packed_panels(rows) * ((cols + 127) / 128) >= ((int64_t)1 << 31))
        return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q_col) || (col_packed && !aligned16(s_col)) ||
        (q_row_packed && (!aligned16(q_row_packed) || !aligned16(s_row_packed))) || ((uintptr_t)src_offsets & 3u) ||
        ((uintptr_t)dst_offsets & 3u))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_dual_grouped_packed(static_cast<const uint16_t *>(x_bf16), rows, cols, q_row_packed,
                                                      s_row_packed, q_col, s_col, col_packed, src_offsets, dst_offsets,
                                                      G, rows_out, stream));
}

mxfp8_status mxfp8_quantize_packed(const void *w_bf16, int64_t batch, int64_t rows, int64_t cols,
                                   uint8_t *q, uint8_t *scales, uint8_t *q_packed,
                                   uint8_t *scales_packed, hipStream_t stream) {
    if (!w_bf16 || !q_packed || !scales_packed) return MXFP8_ERR_NULL;
    if ((q == nullptr) != (scales == nullptr)) return MXFP8_ERR_NULL;
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 32) return MXFP8_ERR_SHAPE;
    if (rows >= kMaxDim || cols > kMaxK || batch > 65535 || !repack_tiles_ok(batch, rows, cols))
        return MXFP8_ERR_SHAPE;
    if (!aligned16(w_bf16) || !aligned16(q_packed) || !aligned16(scales_packed) ||
        (q && (!aligned16(q) || !aligned16(scales))))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_packed(static_cast<const uint16_t *>(w_bf16), batch, rows, cols,
                                         q, scales, q_packed, scales_packed, stream));
}

mxfp8_status mxfp8_quantize_packed_axis0(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols,
                                         uint8_t *q_packed, uint8_t *scales_packed, hipStream_t stream) {
    if (!x_bf16 || !q_packed || !scales_packed) return MXFP8_ERR_NULL;
    if (batch <= 0 || rows <= 0 || cols <= 0 || rows % 32 || cols % 8) return MXFP8_ERR_SHAPE;
    if (cols >= kMaxDim || rows > kMaxK || batch > 65535 || !repack_tiles_ok(batch, cols, rows))
        return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(q_packed) || !aligned16(scales_packed)) return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_axis0_packed(static_cast<const uint16_t *>(x_bf16), batch, rows, cols,
                                               q_packed, scales_packed, stream));
}

mxfp8_status mxfp8_quantize_many(const mxfp8_quant_job *jobs, int64_t count, hipStream_t stream) {
    if (!jobs) return MXFP8_ERR_NULL;
    if (count < 1 || count > MXFP8_QUANT_JOBS_MAX) return MXFP8_ERR_SHAPE;
    static_assert(MXFP8_QUANT_JOBS_MAX == kQuantJobsMax, "job table size");
    QuantJobs t = {};
    int64_t steps = 0;
    for (int64_t i = 0; i < count; ++i) {
        const mxfp8_quant_job &j = jobs[i];
        if (!j.x_bf16 || !j.q || !j.scales) return MXFP8_ERR_NULL;
        if (j.rows <= 0 || j.cols <= 0 || j.rows >= kMaxDim || j.cols >= kMaxDim || j.cols % 32)
            return MXFP8_ERR_SHAPE;
        if (!aligned16(j.x_bf16) || !aligned16(j.q) || !aligned16(j.scales)) return MXFP8_ERR_ALIGN;
        const int64_t nblocks = j.rows * (j.cols / 32);
        steps += (nblocks + 63) / 64;
        if (steps >= ((int64_t)1 << 40)) return MXFP8_ERR_SHAPE;
        t.x[i] = static_cast<const uint16_t *>(j.x_bf16);
        t.q[i] = j.q;
        t.s[i] = j.scales;
        t.nblocks[i] = nblocks;
        t.step_end[i] = steps;
    }
    t.count = (int)count;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_many(t, stream));
}

mxfp8_status mxfp8_quantize_many_layouts(const mxfp8_quant_layout_job *jobs, int64_t count,
                                         hipStream_t stream) {
    if (!jobs) return MXFP8_ERR_NULL;
    if (count < 1 || count > MXFP8_QUANT_JOBS_MAX) return MXFP8_ERR_SHAPE;
    QuantJobs t = {};
    int64_t steps = 0;
    for (int64_t i = 0; i < count; ++i) {
        const mxfp8_quant_layout_job &j = jobs[i];
        if (!j.x_bf16 || !j.q || !j.scales) return MXFP8_ERR_NULL;
        const int lay = raw(j.layout);
        if (lay != MXFP8_CANONICAL && lay != MXFP8_PACKED) return MXFP8_ERR_DTYPE;
        if (j.rows <= 0 || j.cols <= 0 || j.rows >= kMaxDim || j.cols >= kMaxDim || j.cols % 32)
            return MXFP8_ERR_SHAPE;
        if (!aligned16(j.x_bf16) || !aligned16(j.q) || !aligned16(j.scales)) return MXFP8_ERR_ALIGN;
        const int64_t nblocks = j.rows * (j.cols / 32);
        int64_t s;
        if (lay == MXFP8_PACKED) {
            if (j.cols > kMaxK || !repack_tiles_ok(1, j.rows, j.cols)) return MXFP8_ERR_SHAPE;
            s = packed_panels(j.rows) * 16 * packed_ksteps(j.cols);
            if (s >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
        } else {
            s = (nblocks + 63) / 64;
        }
        steps += s;
        if (steps >= ((int64_t)1 << 40)) return MXFP8_ERR_SHAPE;
        t.x[i] = static_cast<const uint16_t *>(j.x_bf16);
        t.q[i] = j.q;
        t.s[i] = j.scales;
        t.nblocks[i] = nblocks;
        t.step_end[i] = steps;
        t.rows[i] = j.rows;
        t.cols[i] = j.cols;
        t.packed[i] = lay == MXFP8_PACKED;
    }
    t.count = (int)count;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_many(t, stream));
}

mxfp8_status mxfp8_quantize_packed_many(const mxfp8_packed_job *jobs, int64_t count,
                                        hipStream_t stream) {
    if (!jobs) return MXFP8_ERR_NULL;
    if (count < 1 || count > MXFP8_PACKED_JOBS_MAX) return MXFP8_ERR_SHAPE;
    static_assert(MXFP8_PACKED_JOBS_MAX == kPackedJobsMax, "job table size");
    PackedJobs t = {};
    int64_t tiles = 0;
    for (int64_t i = 0; i < count; ++i) {
        const mxfp8_packed_job &j = jobs[i];
        if (!j.w_bf16) return MXFP8_ERR_NULL;
        if ((j.q == nullptr) != (j.scales == nullptr)) return MXFP8_ERR_NULL;
        if ((j.q_packed == nullptr) != (j.scales_packed == nullptr)) return MXFP8_ERR_NULL;
        if (!j.q && !j.q_packed) return MXFP8_ERR_NULL;        // no output at all
        if (j.batch <= 0 || j.rows <= 0 || j.cols <= 0 || j.cols % 32) return MXFP8_ERR_SHAPE;
        if (j.rows >= kMaxDim || j.cols > kMaxK || j.batch > 65535 ||
            !repack_tiles_ok(j.batch, j.rows, j.cols))
            return MXFP8_ERR_SHAPE;
        if (!aligned16(j.w_bf16) || (j.q_packed && (!aligned16(j.q_packed) || !aligned16(j.scales_packed))) ||
            (j.q && (!aligned16(j.q) || !aligned16(j.scales))))
            return MXFP8_ERR_ALIGN;
        tiles += j.batch * packed_panels(j.rows) * packed_ksteps(j.cols);
        if (tiles >= ((int64_t)1 << 24)) return MXFP8_ERR_SHAPE;
        t.w[i] = static_cast<const uint16_t *>(j.w_bf16);
        t.qc[i] = j.q;
        t.sc[i] = j.scales;
        t.qp[i] = j.q_packed;
        t.sp[i] = reinterpret_cast<uint32_t *>(j.scales_packed);
        t.N[i] = j.rows;
        t.K[i] = j.cols;
        t.tile_end[i] = tiles;
    }
    t.count = (int)count;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_quantize_packed_jobs(t, stream));
}

size_t mxfp8_selfcheck_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K < 32 || K % 32 || M > kMaxSelfcheckRows || N >= kMaxDim || K > kMaxK)
        return 0;
    return (size_t)selfcheck_workspace(M, N, K).total;
}

mxfp8_status mxfp8_selfcheck(const void *x_bf16, int64_t M, int64_t N, int64_t K,
                             const uint8_t *w_q, const uint8_t *w_s, const uint8_t *w_q_packed,
                             const uint8_t *w_s_packed, void *workspace, double *d_result,
                             hipStream_t stream) {
    if (!x_bf16 || !w_q || !w_s || !w_q_packed || !w_s_packed || !workspace || !d_result)
        return MXFP8_ERR_NULL;
    if (M <= 0 || N <= 0 || K < 32 || K % 32 || M > kMaxSelfcheckRows || N >= kMaxDim || K > kMaxK)
        return MXFP8_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(w_q_packed) ||
        !aligned16(w_s_packed) || !aligned16(workspace) || ((uintptr_t)d_result & 7u))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    const SelfcheckWorkspace ws = selfcheck_workspace(M, N, K);
    uint8_t *base = static_cast<uint8_t *>(workspace);
    uint8_t *xq = base + ws.xq, *xs = base + ws.xs;
    float *y = reinterpret_cast<float *>(base + ws.y);
    float *yref = reinterpret_cast<float *>(base + ws.yref);
    double *part = reinterpret_cast<double *>(base + ws.part);
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    // the serving path: quantize the probe, MXFP8 GEMM against the packed storage
    hipError_t e = launch_quantize(x, M, K, 1, xq, xs, stream);
    if (e == hipSuccess)
        e = launch_gemm(xq, xs, w_q_packed, w_s_packed, true, M, N, K, y, false, stream);
    // the reference from the canonical synchronized grid, then the error
    if (e == hipSuccess) e = launch_selfcheck_ref(x, M, N, K, w_q, w_s, yref, stream);
    if (e == hipSuccess) e = launch_selfcheck_error(y, yref, M * N, part, d_result, stream);
    return finish(e);
}

mxfp8_status mxfp8_dequantize(const uint8_t *q, const uint8_t *scales, int64_t rows, int64_t cols,
                              int axis, void *out, mxfp8_dtype out_dtype, hipStream_t stream) {
    if (!q || !scales || !out) return MXFP8_ERR_NULL;
    if (axis != 0 && axis != 1) return MXFP8_ERR_AXIS;
    if (raw(out_dtype) != MXFP8_F32 && raw(out_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (rows <= 0 || cols <= 0 || rows >= kMaxDim || cols >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (axis == 1 && cols % 32) return MXFP8_ERR_SHAPE;
    if (axis == 0 && (rows % 32 || (rows + 63) / 64 > 65535)) return MXFP8_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(out)) return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_dequantize(q, scales, rows, cols, axis, out, raw(out_dtype) == MXFP8_BF16,
                                    stream));
}

size_t mxfp8_packed_bytes(int64_t batch, int64_t rows, int64_t cols, int which) {
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 32 || (which != 0 && which != 1)) return 0;
    if (rows >= kMaxDim || cols > kMaxK || batch > 65535 || !repack_tiles_ok(batch, rows, cols))
        return 0;
    return (size_t)(which == 0 ? packed_q_bytes(batch, rows, cols) : packed_s_bytes(batch, rows, cols));
}

mxfp8_status mxfp8_repack(const uint8_t *q, const uint8_t *scales, int64_t batch, int64_t rows,
                          int64_t cols, uint8_t *q_packed, uint8_t *scales_packed,
                          hipStream_t stream) {
    if (!q || !scales || !q_packed || !scales_packed) return MXFP8_ERR_NULL;
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 32) return MXFP8_ERR_SHAPE;
    if (rows >= kMaxDim || cols > kMaxK || batch > 65535 || !repack_tiles_ok(batch, rows, cols))
        return MXFP8_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(scales) || !aligned16(q_packed) || !aligned16(scales_packed))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_repack(q, scales, batch, rows, cols, q_packed, scales_packed, stream));
}

mxfp8_status mxfp8_gemm(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                        const uint8_t *b_s, mxfp8_layout b_layout, int64_t M, int64_t N, int64_t K,
                        void *c, mxfp8_dtype c_dtype, hipStream_t stream) {
    if (!a_q || !a_s || !b_q || !b_s || !c) return MXFP8_ERR_NULL;
    if (raw(b_layout) != MXFP8_CANONICAL && raw(b_layout) != MXFP8_PACKED) return MXFP8_ERR_DTYPE;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K < 32 || K % 32 || K > kMaxK || M >= kMaxDim || N >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    // tile counts must fit the 1-D grid
    if (ceil_div(M, 256) * ceil_div(N, 128) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q) || !aligned16(b_s) || !aligned16(c))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_gemm(a_q, a_s, b_q, b_s, raw(b_layout) == MXFP8_PACKED, M, N, K, c,
                              raw(c_dtype) == MXFP8_BF16, stream));
}

// A split plan cut down to the slices `workspace` holds (fewer than two: no
// split).
static SplitPlan fit_split(SplitPlan sp, int64_t M, int64_t N, int64_t K, const void *workspace,
                           size_t workspace_bytes) {
    if (sp.splits > 1 && (!workspace || workspace_bytes < (size_t)sp.workspace_bytes)) {
        const int64_t slice = (M * N + 3) / 4 * 4 * 4;
        const int64_t fit = workspace ? (int64_t)(workspace_bytes / (size_t)slice) : 0;
        if (fit >= 2) {
            const int64_t ks = ceil_div(K, 128);
            const int64_t steps = ceil_div(ks, fit);
            sp.split_steps = (int)steps;
            sp.splits = (int)ceil_div(ks, steps);
            sp.workspace_bytes = sp.splits * slice;
        } else {
            sp.splits = 1;
        }
    }
    return sp;
}

mxfp8_status mxfp8_gemm_packed(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q, const uint8_t *b_s,
                               int64_t M, int64_t N, int64_t K, void *c, mxfp8_dtype c_dtype,
                               hipStream_t stream) {
    if (!a_q || !a_s || !b_q || !b_s || !c) return MXFP8_ERR_NULL;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K < 128 || K % 128 || K > kMaxK || M >= kMaxDim || N >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    if (ceil_div(M, 256) * ceil_div(N, 128) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q) || !aligned16(b_s) || !aligned16(c))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_gemm_packed(a_q, a_s, b_q, b_s, M, N, K, c, raw(c_dtype) == MXFP8_BF16, stream));
}

mxfp8_status mxfp8_gemm_packed_splitk(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                      const uint8_t *b_s, int64_t M, int64_t N, int64_t K, void *c,
                                      mxfp8_dtype c_dtype, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    if (!a_q || !a_s || !b_q || !b_s || !c) return MXFP8_ERR_NULL;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K < 128 || K % 128 || K > kMaxK || M >= kMaxDim || N >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    if (ceil_div(M, 256) * ceil_div(N, 128) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q) || !aligned16(b_s) || !aligned16(c) ||
        (workspace && !aligned16(workspace)))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    const int cus = device_cu_count();
    SplitPlan sp = fit_split(splitk_plan(M, N, K, cus), M, N, K, workspace, workspace_bytes);
    // the split launch stores fp32 partials in 4-column pieces
    if (N % 4 != 0 || (int64_t)128 * N * 4 >= ((int64_t)1 << 31)) sp.splits = 1;
    // 128-row tiles that keep at least half the CUs busy over at most 64
    // k-steps: unsplit, without the partial stores and the reduce pass
    if (packed_tiling(M, N, raw(c_dtype) == MXFP8_BF16, cus) == PackedTiling::kWsHalf &&
        2 * ceil_div(M, 128) * ceil_div(N, 128) >= cus && ceil_div(K, 128) <= 64)
        sp.splits = 1;
    if (sp.splits <= 1)
        return finish(launch_gemm_packed(a_q, a_s, b_q, b_s, M, N, K, c, raw(c_dtype) == MXFP8_BF16, stream));
    return finish(launch_gemm_packed_splitk(a_q, a_s, b_q, b_s, M, N, K, c, raw(c_dtype) == MXFP8_BF16, sp,
                                            static_cast<float *>(workspace), stream));
}

mxfp8_status mxfp8_gemm_accurate(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                 const uint8_t *b_s, mxfp8_layout b_layout, int64_t M, int64_t N, int64_t K,
                                 void *c, mxfp8_dtype c_dtype, hipStream_t stream) {
    if (!a_q || !a_s || !b_q || !b_s || !c) return MXFP8_ERR_NULL;
    if (raw(b_layout) != MXFP8_CANONICAL && raw(b_layout) != MXFP8_PACKED) return MXFP8_ERR_DTYPE;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K < 32 || K % 32 || K > kMaxK || M >= kMaxDim || N >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    if (ceil_div(M, 256) * ceil_div(N, 128) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q) || !aligned16(b_s) || !aligned16(c))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    return finish(launch_gemm_accurate(a_q, a_s, b_q, b_s, raw(b_layout) == MXFP8_PACKED, M, N, K, c,
                                       raw(c_dtype) == MXFP8_BF16, stream));
}

size_t mxfp8_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K < 32 || K % 32 || K > kMaxK || M >= kMaxDim || N >= kMaxDim) return 0;
    if (check_device() != MXFP8_OK) return 0;
    const SplitPlan sp = splitk_plan(M, N, K, device_cu_count());
    return sp.splits > 1 ? (size_t)sp.workspace_bytes : 0;
}

mxfp8_status mxfp8_gemm_splitk(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                               const uint8_t *b_s, mxfp8_layout b_layout, int64_t M, int64_t N, int64_t K,
                               void *c, mxfp8_dtype c_dtype, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (!a_q || !a_s || !b_q || !b_s || !c) return MXFP8_ERR_NULL;
    if (raw(b_layout) != MXFP8_CANONICAL && raw(b_layout) != MXFP8_PACKED) return MXFP8_ERR_DTYPE;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K < 32 || K % 32 || K > kMaxK || M >= kMaxDim || N >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    if (ceil_div(M, 256) * ceil_div(N, 128) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q) || !aligned16(b_s) || !aligned16(c) ||
        (workspace && !aligned16(workspace)))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    const SplitPlan sp = fit_split(splitk_plan(M, N, K, device_cu_count()), M, N, K, workspace, workspace_bytes);
    if (sp.splits <= 1)
        return finish(launch_gemm(a_q, a_s, b_q, b_s, raw(b_layout) == MXFP8_PACKED, M, N, K, c,
                                  raw(c_dtype) == MXFP8_BF16, stream));
    return finish(launch_gemm_splitk(a_q, a_s, b_q, b_s, raw(b_layout) == MXFP8_PACKED, M, N, K, c,
                                     raw(c_dtype) == MXFP8_BF16, sp, static_cast<float *>(workspace), stream));
}

mxfp8_status mxfp8_gemm_splitk_noalloc(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                                       const uint8_t *b_s, mxfp8_layout b_layout, int64_t M, int64_t N,
                                       int64_t K, void *c, mxfp8_dtype c_dtype, hipStream_t stream) {
    if (!a_q || !a_s || !b_q || !b_s || !c) return MXFP8_ERR_NULL;
    if (raw(b_layout) != MXFP8_CANONICAL && raw(b_layout) != MXFP8_PACKED) return MXFP8_ERR_DTYPE;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K < 32 || K % 32 || K > kMaxK || M >= kMaxDim || N >= kMaxDim)
        return MXFP8_ERR_SHAPE;
    if (ceil_div(M, 256) * ceil_div(N, 128) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q) || !aligned16(b_s) || !aligned16(c))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    const SplitPlan sp = splitk_plan(M, N, K, device_cu_count());
    if (sp.splits <= 1)
        return finish(launch_gemm(a_q, a_s, b_q, b_s, raw(b_layout) == MXFP8_PACKED, M, N, K, c,
                                  raw(c_dtype) == MXFP8_BF16, stream));
    void *ws = nullptr;
    size_t ws_bytes = 0;
    const hipError_t e = splitk_scratch(&ws, &ws_bytes);
    if (e != hipSuccess) return finish(e);
    if ((size_t)sp.workspace_bytes > ws_bytes) return MXFP8_ERR_SHAPE;   // plan exceeds the static scratch
    return finish(launch_gemm_splitk(a_q, a_s, b_q, b_s, raw(b_layout) == MXFP8_PACKED, M, N, K, c,
                                     raw(c_dtype) == MXFP8_BF16, sp, static_cast<float *>(ws), stream));
}

mxfp8_status mxfp8_grouped_gemm(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q_packed,
                                const uint8_t *b_s_packed, const int32_t *d_group_offsets,
                                int64_t G, int64_t M_total, int64_t N, int64_t K, void *c,
                                mxfp8_dtype c_dtype, hipStream_t stream) {
    if (!a_q || !a_s || !b_q_packed || !b_s_packed || !d_group_offsets || !c) return MXFP8_ERR_NULL;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (G < 1 || G > 65535 || M_total < 0 || M_total % 32 || M_total >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (N <= 0 || N >= kMaxDim || K < 32 || K % 32 || K > kMaxK) return MXFP8_ERR_SHAPE;
    if ((ceil_div(M_total, 128) + G) * ceil_div(N, 256) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(b_q_packed) || !aligned16(b_s_packed) ||
        !aligned16(c))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    if (M_total == 0) return MXFP8_OK;
    return finish(launch_grouped_gemm(a_q, a_s, b_q_packed, b_s_packed, d_group_offsets, G,
                                      M_total, N, K, c, raw(c_dtype) == MXFP8_BF16, stream));
}

mxfp8_status mxfp8_grouped_gemm_packed(const uint8_t *a_q_packed, const uint8_t *a_s_packed,
                                       const uint8_t *b_q_packed, const uint8_t *b_s_packed,
                                       const int32_t *d_group_offsets, int64_t G, int64_t M_total, int64_t N,
                                       int64_t K, void *c, mxfp8_dtype c_dtype, hipStream_t stream) {
    if (!a_q_packed || !a_s_packed || !b_q_packed || !b_s_packed || !d_group_offsets || !c) return MXFP8_ERR_NULL;
    if (raw(c_dtype) != MXFP8_F32 && raw(c_dtype) != MXFP8_BF16) return MXFP8_ERR_DTYPE;
    if (G < 1 || G > 65535 || M_total < 0 || M_total % 32 || M_total >= kMaxDim) return MXFP8_ERR_SHAPE;
    if (N <= 0 || N >= kMaxDim || K < 128 || K % 128 || K > kMaxK) return MXFP8_ERR_SHAPE;
    if ((ceil_div(M_total, 256) + G) * ceil_div(N, 256) >= ((int64_t)1 << 31)) return MXFP8_ERR_SHAPE;
    if (!aligned16(a_q_packed) || !aligned16(a_s_packed) || !aligned16(b_q_packed) || !aligned16(b_s_packed) ||
        !aligned16(c))
        return MXFP8_ERR_ALIGN;
    mxfp8_status st = check_device();
    if (st != MXFP8_OK) return st;
    if (M_total == 0) return MXFP8_OK;
    return finish(launch_grouped_gemm_packed(a_q_packed, a_s_packed, b_q_packed, b_s_packed, d_group_offsets, G,
                                             M_total, N, K, c, raw(c_dtype) == MXFP8_BF16, stream));
}

}  // extern "C"
