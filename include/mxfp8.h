/*
 * mxfp8.h -- C ABI of the MI355X (gfx950) MXFP8 library.
 *
 * The number format is the one described on the page "End-to-End MXFP8 RL on
 * Blackwell: What Matching Buys, When It Pays Off, and How It Fails" (verl
 * blog), section "The pipeline", paragraph "The format", which follows the
 * OCP Microscaling (MX) v1.0 specification: every run of 32 consecutive
 * values along the axis a GEMM sums over is stored as 32 one-byte E4M3
 * codes plus a single one-byte E8M0 power-of-two multiplier, so a tensor
 * costs 8 + 8/32 bits per value.
 *
 * Conventions shared by every call
 *  - All matrices are row-major.  BF16 inputs are raw 16-bit patterns.
 *  - Device pointers (all tensors, the group offsets) must be device memory
 *    that the stream's device can access, 16-byte aligned.
 *  - The caller allocates and owns every buffer.  The library never
 *    allocates, frees, copies to the host or synchronizes: every call only
 *    validates its arguments on the host and enqueues kernels on `stream`
 *    (0 = the legacy default stream), so calls are HIP-graph capturable.
 *  - Arguments are validated before anything is enqueued; on a validation
 *    error nothing is written and a non-zero status is returned.  A failed
 *    launch returns MXFP8_ERR_HIP (mxfp8_last_hip_error() gives the HIP
 *    code).  Faults inside a kernel surface at the caller's next
 *    synchronization of the stream, as for any asynchronous HIP work.
 *  - Calls are thread-safe; the library keeps no mutable global state
 *    except the last HIP error code (per thread).
 *  - Outputs are deterministic: the same inputs give the same bytes.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXFP8_OK = 0,
    MXFP8_ERR_NULL = 1,        /* a required pointer is NULL                          */
    MXFP8_ERR_SHAPE = 2,       /* a size <= 0 (or < 0 where 0 is allowed), a block
                                  axis not a multiple of 32, or a size too large     */
    MXFP8_ERR_AXIS = 3,        /* axis is not 0 or 1                                  */
    MXFP8_ERR_DTYPE = 4,       /* unknown output dtype or B layout                    */
    MXFP8_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                    */
    MXFP8_ERR_HIP = 6,         /* a HIP launch or query failed                        */
    MXFP8_ERR_UNSUPPORTED = 7  /* the current device is not gfx950                    */
} mxfp8_status;

typedef enum { MXFP8_F32 = 0, MXFP8_BF16 = 1 } mxfp8_dtype;

typedef enum { MXFP8_CANONICAL = 0, MXFP8_PACKED = 1 } mxfp8_layout;

/*
 * mxfp8_quantize -- BF16 -> MXFP8 (E4M3 elements + one E8M0 scale per 32).
 *
 * Defined by the format paragraph above (blocks of 32 along the reduction
 * axis) and, for axis 0, by the learner paragraph of the same section: the
 * weight-gradient GEMM reduces over tokens, so some operands are blocked in
 * 32s along the token dimension.
 *
 * Per block of 32 BF16 values x_i:
 *   amax = max |x_i|; scale exponent s = floor(log2 amax) - 8 (OCP MX rule,
 *   8 = largest exponent of E4M3), clamped to s >= -127; scale code = s+127.
 *   An all-zero block has code 0; a block holding any NaN or +-Inf has
 *   code 0xFF and all its elements 0x7F.  BF16 subnormals are not flushed.
 *   q_i = x_i * 2^-s rounded to the nearest E4M3 value (ties to even),
 *   saturated to +-448; the sign of zero is kept.
 *
 *   x      : BF16 [rows][cols]
 *   axis 1 : blocks along cols.  cols % 32 == 0.
 *            q[rows][cols], scales[rows][cols/32]
 *   axis 0 : blocks along rows (tokens).  rows % 32 == 0.  The output is
 *            TRANSPOSED so the block axis is contiguous (every GEMM operand
 *            is then K-contiguous):  q[cols][rows], scales[cols][rows/32].
 * rows, cols >= 1.  Bit-exact and deterministic.
 */
mxfp8_status mxfp8_quantize(const void *x_bf16, int64_t rows, int64_t cols,
                            int axis, uint8_t *q, uint8_t *scales,
                            hipStream_t stream);

/*
 * mxfp8_quantize_dual -- one BF16 read, both operand grids of a learner tensor.
 *
 * The learner quantizes the operands of each linear layer's three GEMMs on
 * the fly, and because the weight-gradient GEMM reduces over tokens some
 * operands are blocked along tokens ("The pipeline", learner paragraph); the
 * page counts the activation and gradient quantize launches per micro-batch
 * among its added costs (section "Speed: when it pays off", "Where the time
 * goes").  An activation or gradient feeds one GEMM blocked along its columns
 * and another blocked along its rows; this call writes both from a single
 * read (4.0625 instead of 6.0625 HBM bytes per element).
 *
 * Result: byte-for-byte mxfp8_quantize(x, axis=1) into (q_row, s_row) and
 * mxfp8_quantize(x, axis=0) into (q_col, s_col):
 *   q_row[rows][cols], s_row[rows][cols/32], q_col[cols][rows], s_col[cols][rows/32].
 * rows % 32 == 0, cols % 32 == 0, rows, cols >= 32.  Bit-exact, deterministic.
 */
mxfp8_status mxfp8_quantize_dual(const void *x_bf16, int64_t rows, int64_t cols,
                                 uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                                 uint8_t *s_col, hipStream_t stream);

/*
 * mxfp8_quantize_dual_packed -- mxfp8_quantize_dual with both grids written
 * straight into the GEMM's packed operand layout.
 *
 * The learner's activations and output gradients feed three GEMMs each:
 * blocked along K (forward and data gradient) and along tokens, transposed
 * (weight gradient); its weights feed the forward GEMM blocked along K and
 * the data-gradient GEMM blocked along N ("The pipeline", learner
 * paragraph).  One BF16 read of x[batch][rows][cols] (rows % 32 == 0,
 * cols % 32 == 0; 1 <= batch <= 65535, e.g. the experts of an MoE layer)
 * writes exactly the bytes mxfp8_repack writes for
 *   q_row_packed / s_row_packed: the axis-1 grids q[b][rows][cols] (N =
 *     rows, K = cols; mxfp8_packed_bytes(batch, rows, cols, 0 / 1) bytes),
 *   q_col_packed / s_col_packed: the axis-0 grids q[b][cols][rows] (N =
 *     cols, K = rows; mxfp8_packed_bytes(batch, cols, rows, 0 / 1) bytes),
 * padding included, so both go to mxfp8_gemm_packed / mxfp8_gemm_packed_splitk
 * (batch 1) or mxfp8_grouped_gemm as A or B.  The limits of mxfp8_repack
 * apply to both layouts.  Bit-exact, deterministic; no allocation, no
 * synchronization.
 */
mxfp8_status mxfp8_quantize_dual_packed(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols,
                                        uint8_t *q_row_packed, uint8_t *s_row_packed,
                                        uint8_t *q_col_packed, uint8_t *s_col_packed, hipStream_t stream);

/*
 * mxfp8_quantize_dual_grouped -- mxfp8_quantize_dual for token-sorted MoE
 * tensors, with the token-blocked grid regrouped for the experts' weight
 * gradients.
 *
 * The expert weight gradient reduces over each expert's own tokens ("The
 * pipeline", learner paragraph: token-axis blocks, groups padded to 32).
 * Giving every expert's token range in the token-blocked (axis-0) grid a
 * start and a length that are multiples of 128 (one 128-deep k-step of the
 * weight-gradient GEMM) lets that GEMM take its aligned path, so the extra
 * padding lives only in this grid.
 *
 * x [rows][cols] BF16, rows sorted by group: group g owns source rows
 * [src_offsets[g], src_offsets[g+1]).  Result:
 *   (q_row, s_row), optional (both NULL or both given): exactly
 *     mxfp8_quantize(x, axis=1);
 *   (q_col, s_col) [cols][rows_out] / [cols][rows_out/32]: exactly
 *     mxfp8_quantize(x', axis=0), where x' [rows_out][cols] holds group g's
 *     source rows at rows [dst_offsets[g], dst_offsets[g] + len_g) and zero
 *     rows everywhere else (so pad blocks have zero codes and scale code 0).
 * src_offsets, dst_offsets: DEVICE int32 [G+1], read on the device (no host
 * synchronization).  Well-formed tables: both non-decreasing, multiples of
 * 32, dst_offsets[g+1] - dst_offsets[g] >= len_g, src within [0, rows], dst
 * within [0, rows_out].  Others are clamped like mxfp8_grouped_gemm's
 * (a group's block goes nowhere unless both of its starts are multiples of
 * 32 and the block fits its destination range); they can leave bytes of
 * q_col unspecified but never address outside the buffers.
 * rows % 32 == 0, cols % 32 == 0, rows_out % 32 == 0, 1 <= G <= 65535.
 * x, q_row, s_row and q_col 16-byte aligned, offsets 4-byte aligned.
 * Bit-exact, deterministic for well-formed tables.
 */
mxfp8_status mxfp8_quantize_dual_grouped(const void *x_bf16, int64_t rows, int64_t cols,
                                         uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                                         uint8_t *s_col, const int32_t *src_offsets,
                                         const int32_t *dst_offsets, int64_t G, int64_t rows_out,
                                         hipStream_t stream);

/*
 * mxfp8_quantize_dual_grouped_packed -- mxfp8_quantize_dual_grouped with the
 * row grid written straight into the GEMM's packed operand layout, and the
 * regrouped token-blocked grid in the layout the caller picks.
 *
 * One BF16 read of the token-sorted x [rows][cols] gives
 *   q_row_packed / s_row_packed (optional: both NULL or both given): the
 *     operand of the experts' forward or data-gradient GEMM
 *     (mxfp8_grouped_gemm_packed's A), exactly what mxfp8_repack writes for
 *     mxfp8_quantize(x, axis=1) with N = rows, K = cols
 *     (mxfp8_packed_bytes(1, rows, cols, 0 / 1) bytes, padding included);
 *   q_col / s_col: the regrouped token-blocked grid of the experts' weight
 *     gradients -- col_layout MXFP8_CANONICAL: exactly
 *     mxfp8_quantize_dual_grouped's (q_col, s_col) (for
 *     mxfp8_grouped_gemm_wgrad); MXFP8_PACKED: exactly what mxfp8_repack
 *     writes for that grid with N = cols, K = rows_out
 *     (mxfp8_packed_bytes(1, cols, rows_out, 0 / 1) bytes; pad blocks zero
 *     codes with scale code 0, the layout's padding scale code 127; for
 *     mxfp8_grouped_gemm_wgrad_packed).
 * Arguments, table rules and limits as mxfp8_quantize_dual_grouped, plus
 * those of mxfp8_repack for the packed layouts (s_col 16-byte aligned only
 * when packed); MXFP8_ERR_DTYPE for a col_layout other than the two.
 * Bit-exact, deterministic; no allocation, no synchronization.
 */
mxfp8_status mxfp8_quantize_dual_grouped_packed(const void *x_bf16, int64_t rows, int64_t cols,
                                                uint8_t *q_row_packed, uint8_t *s_row_packed,
                                                uint8_t *q_col, uint8_t *s_col, mxfp8_layout col_layout,
                                                const int32_t *src_offsets, const int32_t *dst_offsets,
                                                int64_t G, int64_t rows_out, hipStream_t stream);

/*
 * mxfp8_quantize_packed -- weights BF16 -> MXFP8 straight into the GEMM's
 * packed layout, optionally also the canonical grid.
 *
 * The weight synchronization passes every weight through the learner's
 * forward-weight quantizer, and the sampler then rebuilds its kernel layouts
 * from the result ("The pipeline", weight-synchronization and sampler
 * paragraphs; writing cached weights' scales directly in the GEMM's layout is
 * the remedy the page notes under "Speed: when it pays off", "Where the time
 * goes").  This call is quantize(axis 1) followed by repack in one pass:
 *   q_packed / scales_packed: exactly what mxfp8_repack writes for the
 *     canonical result (sizes from mxfp8_packed_bytes);
 *   q / scales (both NULL or both given): exactly mxfp8_quantize(w, axis=1),
 *     q[batch][rows][cols], scales[batch][rows][cols/32].
 * w is BF16 [batch][rows=N][cols=K]; the limits of mxfp8_repack apply.
 * HBM bytes per element: 3.03125 packed only, 4.0625 with the canonical grid
 * (quantize + repack: 5.09375).  Bit-exact, deterministic; writes in place,
 * so graph-captured pointers stay valid.
 */
mxfp8_status mxfp8_quantize_packed(const void *w_bf16, int64_t batch, int64_t rows,
                                   int64_t cols, uint8_t *q, uint8_t *scales,
                                   uint8_t *q_packed, uint8_t *scales_packed,
                                   hipStream_t stream);

/* One tensor of an mxfp8_quantize_many call: the arguments of
 * mxfp8_quantize(x, rows, cols, axis = 1, q, scales) for that tensor. */
typedef struct {
    const void *x_bf16;        /* BF16 [rows][cols]                                */
    int64_t rows, cols;
    uint8_t *q, *scales;       /* q[rows][cols], scales[rows][cols/32]             */
} mxfp8_quant_job;

#define MXFP8_QUANT_JOBS_MAX 8

/*
 * mxfp8_quantize_many -- mxfp8_quantize along axis 1 over a list of tensors
 * in one launch.
 *
 * A linear layer's forward quantizes its weights and its activations along
 * the reduction axis (format paragraph of "The pipeline"); one launch for
 * both pays one launch ramp and tail instead of two.  jobs: HOST array of
 * `count` entries (1 <= count <= MXFP8_QUANT_JOBS_MAX), each validated as
 * mxfp8_quantize(axis = 1) validates its arguments; the wave-steps of all
 * entries together (ceil(rows * cols / 2048) each) must stay below 2^40.
 * The output of every entry is exactly what mxfp8_quantize(axis = 1) writes
 * for it; entries must not overlap in memory.  The array is read during the
 * call only (passed by value to the kernel).  Bit-exact, deterministic.
 */
mxfp8_status mxfp8_quantize_many(const mxfp8_quant_job *jobs, int64_t count, hipStream_t stream);

/* One tensor of an mxfp8_quantize_many_layouts call: BF16 [rows][cols]
 * quantized along its columns (axis 1) into the given layout. */
typedef struct {
    const void *x_bf16;        /* BF16 [rows][cols]                                */
    int64_t rows, cols;
    mxfp8_layout layout;       /* MXFP8_CANONICAL or MXFP8_PACKED                  */
    uint8_t *q, *scales;       /* canonical: q[rows][cols], scales[rows][cols/32];
                                  packed: the mxfp8_repack layout of that grid
                                  (mxfp8_packed_bytes(1, rows, cols, 0 / 1) bytes) */
} mxfp8_quant_layout_job;

/*
 * mxfp8_quantize_many_layouts -- mxfp8_quantize_many with a layout per
 * tensor.
 *
 * A canonical entry writes exactly what mxfp8_quantize(axis = 1) writes; a
 * packed entry writes exactly the bytes mxfp8_repack writes for that
 * canonical grid (padding rows and blocks included).  Why: a linear layer's
 * activations quantized straight into the GEMM's operand layout for
 * mxfp8_gemm_packed, in the same launch as its weights' canonical grid.  The
 * packed entries are walked in steps of 16 rows x 128 columns, so each
 * step's codes land as 2 KB of one packed tile and its scales as one 64-byte
 * record.  jobs: HOST array of `count` entries (1 <= count <=
 * MXFP8_QUANT_JOBS_MAX), each validated as mxfp8_quantize(axis = 1)
 * validates its arguments, plus: layout one of the two values
 * (MXFP8_ERR_DTYPE), a packed entry's tiles as mxfp8_repack limits them and
 * its steps (ceil(rows / 256) * 16 * ceil(cols / 128)) below 2^31.
 * Entries must not overlap in memory.  The array is read during the call
 * only.  Bit-exact, deterministic.
 */
mxfp8_status mxfp8_quantize_many_layouts(const mxfp8_quant_layout_job *jobs, int64_t count,
                                         hipStream_t stream);

/* One weight of an mxfp8_quantize_packed_many call: the arguments of
 * mxfp8_quantize_packed for that weight. */
typedef struct {
    const void *w_bf16;        /* BF16 [batch][rows][cols]                         */
    int64_t batch, rows, cols;
    uint8_t *q, *scales;       /* canonical grid, or both NULL                     */
    uint8_t *q_packed, *scales_packed;   /* packed layout, or both NULL            */
} mxfp8_packed_job;

#define MXFP8_PACKED_JOBS_MAX 32

/*
 * mxfp8_quantize_packed_many -- mxfp8_quantize_packed over a list of weights
 * in one launch.
 *
 * A weight synchronization quantizes every linear of the model ("The
 * pipeline", weight-synchronization paragraph); one launch per weight pays a
 * launch ramp and tail per weight, which costs most on the smaller
 * projections.  jobs: HOST array of `count` entries (1 <= count <=
 * MXFP8_PACKED_JOBS_MAX), each validated as mxfp8_quantize_packed validates
 * its arguments, except that an entry may leave both packed pointers NULL
 * when it gives the canonical grid (then it writes that grid only; an entry
 * with neither output is MXFP8_ERR_NULL); the tiles of all entries together
 * must stay below 2^24 (batch * ceil(rows/256) * ceil(cols/128) summed over
 * the list).  The output of every entry is exactly what mxfp8_quantize_packed
 * (or, canonical only, mxfp8_quantize(axis = 1)) writes for it; entries
 * must not overlap in memory.  The array is read during the call only (its
 * contents are passed by value to the kernel, so a captured graph keeps
 * them).  Bit-exact, deterministic.
 */
mxfp8_status mxfp8_quantize_packed_many(const mxfp8_packed_job *jobs, int64_t count,
                                        hipStream_t stream);

/*
 * mxfp8_quantize_packed_axis0 -- weights BF16 -> MXFP8 blocked along their
 * rows (axis 0), straight into the GEMM's packed layout of the transposed
 * grid.
 *
 * The data-gradient GEMM of the learner multiplies by the transposed weights,
 * blocked along the weights' output dimension ("The pipeline", learner
 * paragraph), and the sampler-side layouts are rebuilt after every update;
 * this call is mxfp8_quantize_batched(x, axis = 0) followed by mxfp8_repack of
 * its result (N = cols, K = rows) in one pass:
 *   x: BF16 [batch][rows][cols], rows % 32 == 0, cols % 8 == 0;
 *   q_packed / scales_packed: exactly what mxfp8_repack writes for
 *     q[batch][cols][rows], scales[batch][cols][rows/32] (sizes from
 *     mxfp8_packed_bytes(batch, cols, rows, which)), padding included.
 * The limits of mxfp8_repack apply with N = cols, K = rows; batch <= 65535.
 * HBM bytes per element: 3.03125 (quantize along axis 0 + repack: 5.09375).
 * Bit-exact, deterministic; writes in place.
 */
mxfp8_status mxfp8_quantize_packed_axis0(const void *x_bf16, int64_t batch, int64_t rows,
                                         int64_t cols, uint8_t *q_packed, uint8_t *scales_packed,
                                         hipStream_t stream);

/*
 * mxfp8_quantize_batched -- mxfp8_quantize over `batch` matrices at once.
 *
 * The MoE learner's data-gradient GEMM needs every expert's weights blocked
 * along N (axis 0, transposed; "The pipeline", learner paragraph), one
 * matrix per expert.  x: BF16 [batch][rows][cols]; per matrix the result is
 * exactly mxfp8_quantize's: axis 1 -> q[batch][rows][cols],
 * scales[batch][rows][cols/32]; axis 0 -> q[batch][cols][rows],
 * scales[batch][cols][rows/32] (rows % 32 == 0 and rows * cols % 16 == 0).
 * batch <= 65535.  Bit-exact, deterministic.
 */
mxfp8_status mxfp8_quantize_batched(const void *x_bf16, int64_t batch, int64_t rows,
                                    int64_t cols, int axis, uint8_t *q, uint8_t *scales,
                                    hipStream_t stream);

/*
 * mxfp8_quantize_gather -- routing permute, expert padding and the axis-1
 * quantize in one pass.
 *
 * The MoE GEMMs read token rows sorted by expert with each group padded to a
 * multiple of 32 (the pages pad to 32 for the token-blocked operands, and the
 * expert GEMMs consume their inputs reordered by expert).  Output row i is input row
 * d_row_index[i], quantized along its columns; an index outside
 * [0, rows_in) (the padding rows of a group) gives a zero row (scale code 0,
 * elements 0), so the index table can never make it read out of bounds.
 *   x: BF16 [rows_in][cols], cols % 32 == 0; d_row_index: DEVICE int64
 *   [rows_out]; q [rows_out][cols], scales [rows_out][cols/32].
 * Bit-exact: equal to mxfp8_quantize of the gathered, zero-padded matrix.
 */
mxfp8_status mxfp8_quantize_gather(const void *x_bf16, int64_t rows_in, int64_t cols,
                                   const int64_t *d_row_index, int64_t rows_out,
                                   uint8_t *q, uint8_t *scales, hipStream_t stream);

/*
 * mxfp8_quantize_gather_packed -- mxfp8_quantize_gather written straight into
 * the GEMM's packed operand layout (A of mxfp8_grouped_gemm_packed).
 *
 * Same rows as mxfp8_quantize_gather (output row i is input row
 * d_row_index[i], an index outside [0, rows_in) a zero row), but q_packed /
 * s_packed receive exactly what mxfp8_repack writes for that grid with
 * N = rows_out, K = cols (mxfp8_packed_bytes(1, rows_out, cols, 0 / 1)
 * bytes, padding included).  cols % 32 == 0; the limits of mxfp8_repack
 * apply.  Bit-exact, deterministic; no allocation, no synchronization.
 */
mxfp8_status mxfp8_quantize_gather_packed(const void *x_bf16, int64_t rows_in, int64_t cols,
                                          const int64_t *d_row_index, int64_t rows_out, uint8_t *q_packed,
                                          uint8_t *s_packed, hipStream_t stream);

/*
 * mxfp8_dequantize -- MXFP8 -> FP32 or BF16:  out = decode(q) * 2^(code-127).
 *
 * The high-precision reference that the page's post-sync self-check compares
 * the MXFP8 kernel against is built from dequantized weights (section
 * "Correctness: how it fails", "Post-sync self-check").
 *
 * q / scales are laid out as mxfp8_quantize writes them for `axis`; `out` is
 * [rows][cols] in x's orientation.  FP32 output is exact (an E8M0 code above
 * 246 can overflow to +-Inf); BF16 output is rounded to nearest even.  NaN
 * codes (element 0x7F/0xFF or scale 0xFF) give NaN.
 */
mxfp8_status mxfp8_dequantize(const uint8_t *q, const uint8_t *scales,
                              int64_t rows, int64_t cols, int axis, void *out,
                              mxfp8_dtype out_dtype, hipStream_t stream);

/*
 * mxfp8_packed_bytes -- size in bytes of the packed weight buffers for
 * `batch` matrices of [rows=N][cols=K]: which = 0 -> elements, 1 -> scales.
 * Pure host function; returns 0 for sizes mxfp8_repack rejects (K % 32 != 0,
 * a size <= 0, too many tiles).
 */
size_t mxfp8_packed_bytes(int64_t batch, int64_t rows, int64_t cols, int which);

/*
 * mxfp8_repack -- canonical MXFP8 weights -> the GEMM's kernel layout.
 *
 * Per the page (section "The pipeline", sampler paragraph), the serving
 * kernels do not read the canonical grid itself but their own rearranged
 * copies of it (reordered scale bytes, expert weights in a kernel order),
 * and those copies go stale whenever the weights change: they have to be
 * regenerated from the freshly synchronized canonical tensors each time and
 * stored into the same buffers the recorded graphs point at.  This call is that rebuild: run it after every update; it
 * writes in place into the caller's packed buffers, so pointers captured by a
 * HIP graph stay valid.
 *
 * In : q[batch][N][K], scales[batch][N][K/32] (axis-1 quantizer output of
 *      weights [N][K]; K % 32 == 0, N >= 1, batch >= 1, and at most 2^24 - 1
 *      tiles: batch * ceil(N/256) * ceil(K/128) < 2^24, else MXFP8_ERR_SHAPE).
 * Out: q_packed (mxfp8_packed_bytes(batch,N,K,0) bytes) and scales_packed
 *      (mxfp8_packed_bytes(batch,N,K,1) bytes), with this layout:
 *   NP = ceil(N/256) panels of 256 rows, KS = ceil(K/128) k-steps of 128.
 *   elements [batch][NP][KS][256 rows][128 B]: the bytes k = 128*ks + 16c ..
 *     + 15 of row r of the panel form chunk c (0..7), stored at chunk slot
 *     c ^ (r % 8) (the GEMM's LDS image, whose 16-byte fragment reads of 16
 *     rows at one chunk are then bank-conflict free).  Rows >= N and k >= K
 *     hold 0x00.
 *   scales [batch][NP][KS][16 atoms of 16 rows][64 lanes] bytes: byte
 *     (panel, kstep, atom, lane) is the scale of row 256*panel + 16*atom +
 *     (lane % 16), block 4*kstep + (lane / 16) (the byte the GEMM's MFMA lane
 *     `lane` supplies for that 16-row atom).  Rows >= N or blocks >= K/32
 *     hold 127 (1.0).
 */
mxfp8_status mxfp8_repack(const uint8_t *q, const uint8_t *scales,
                          int64_t batch, int64_t rows, int64_t cols,
                          uint8_t *q_packed, uint8_t *scales_packed,
                          hipStream_t stream);

/*
 * mxfp8_gemm -- block-scaled GEMM  C[M][N] = A[M][K] * B[N][K]^T.
 *
 * The format paragraph (section "The pipeline") describes block scales fed
 * to the matrix instruction as operands; here the scaled MFMA of gfx950
 * consumes the E4M3 elements and E8M0 scales directly:
 *   C[m][n] = sum_b 2^(sa[m][b] + sb[n][b] - 254) * sum_{k in block b} a[m][k] b[n][k]
 * accumulated in fp32.  One A*B^T form serves the learner's three GEMMs:
 * forward (X and W blocked along K), data gradient (dY blocked along N, W
 * quantized with axis 0) and weight gradient (dY and X quantized with axis 0,
 * blocked along tokens).
 *
 *   A (a_q, a_s): canonical K-contiguous MXFP8, q[M][K], s[M][K/32] (axis-1
 *                 output, or axis-0 output, which is already transposed).
 *   B (b_q, b_s): b_layout MXFP8_PACKED -> mxfp8_repack output for [N][K];
 *                 MXFP8_CANONICAL -> q[N][K], s[N][K/32] like A.
 *   C           : [M][N], FP32 or BF16 (round to nearest even).
 * M, N >= 1; K >= 32, K % 32 == 0; a_q, a_s, b_q, b_s and c 16-byte aligned.
 * Deterministic (no split-K atomics).
 */
mxfp8_status mxfp8_gemm(const uint8_t *a_q, const uint8_t *a_s,
                        const uint8_t *b_q, const uint8_t *b_s,
                        mxfp8_layout b_layout, int64_t M, int64_t N, int64_t K,
                        void *c, mxfp8_dtype c_dtype, hipStream_t stream);

/*
 * mxfp8_gemm_packed -- mxfp8_gemm with A in the packed layout as well.
 *
 * Same result definition as mxfp8_gemm (bit-identical output for the same
 * operands).  A (a_q, a_s) is the packed layout of q[M][K], s[M][K/32]
 * (the layout mxfp8_repack describes, with M in place of N): written by
 * mxfp8_quantize_packed straight from BF16 activations, or by mxfp8_repack
 * of a canonical grid.  B (b_q, b_s) is packed as for mxfp8_gemm.  Why: the
 * GEMM copies each k-step's operand tiles into LDS 1 KB per instruction; a
 * canonical A tile is gathered 128 bytes from each of 8 rows K bytes apart,
 * which the address unit issues at about half the rate of a contiguous 1 KB
 * (measured on MI355X: 64 KB of such copies per CU take ~1920 clocks to
 * issue against ~920), while every packed copy is contiguous.  Measured:
 * 4096x6144x4096 101-114 -> 92-98 us, 8192x4096x12288 333-343 -> 312-320 us.
 * M, N >= 1; K >= 128, K % 128 == 0; the five pointers 16-byte aligned.
 * MXFP8_ERR_SHAPE otherwise (K % 128 != 0 included).  Deterministic.
 */
mxfp8_status mxfp8_gemm_packed(const uint8_t *a_q, const uint8_t *a_s,
                               const uint8_t *b_q, const uint8_t *b_s,
                               int64_t M, int64_t N, int64_t K,
                               void *c, mxfp8_dtype c_dtype, hipStream_t stream);

/*
 * mxfp8_gemm_accurate -- mxfp8_gemm with every product exact and the sums
 * carried at fp32 accuracy, so |C - C_ref| <= 1e-4 * sum_k |a_k b_k| holds
 * element by element on every input, outlier-dominated rows included.
 *
 * Same operands, layouts, result definition and argument errors as
 * mxfp8_gemm.  Why it exists: the scaled FP8 matrix instruction that
 * mxfp8_gemm uses adds the products of one instruction (128 K values) with
 * about 12 bits relative to its largest product (measured on MI355X: at most
 * 2^-10.8 of it), which exceeds the 1e-4 * sum|ab| bound on rows whose sum
 * is dominated by a few products (1% of x20 outliers at K = 160: 1.013x the
 * bound).  This call instead converts each E4M3 element times its block
 * scale to BF16 (exact for scale codes 3..246; a step whose operands hold a
 * code outside that range takes unscaled BF16 products per block, scaled by
 * 2^(sa + sb - 254) in fp32) and runs the BF16 matrix instruction, whose
 * sums carry fp32 accuracy (measured: at most 2^-20 of the largest product).
 * About half the speed of mxfp8_gemm (the BF16 matrix rate is half the FP8
 * rate).  Limits shared with any fp32 result: products or sums outside
 * fp32's range over- or underflow.  Deterministic.
 */
mxfp8_status mxfp8_gemm_accurate(const uint8_t *a_q, const uint8_t *a_s,
                                 const uint8_t *b_q, const uint8_t *b_s,
                                 mxfp8_layout b_layout, int64_t M, int64_t N, int64_t K,
                                 void *c, mxfp8_dtype c_dtype, hipStream_t stream);

/*
 * mxfp8_gemm_splitk -- mxfp8_gemm for shapes with few output tiles (small M:
 * the page's break-even analysis measures the MXFP8 layers over the tokens
 * per micro-batch, section "Speed: when it pays off").
 *
 * Same operands, result and error bound as mxfp8_gemm; when the shape has
 * too few 256x128 output tiles to fill the device, K is split into slices
 * (multiples of 128, at least 4 k-steps each) whose fp32 partial tiles go to
 * `workspace` and are then summed in slice order into C (deterministic; the
 * summation order differs from mxfp8_gemm's, so results match it within the
 * bound, not bit for bit).
 *   workspace: DEVICE memory owned by the caller, 16-byte aligned, or NULL;
 *     its contents on entry are ignored and on return unspecified.  With
 *     workspace_bytes >= mxfp8_gemm_splitk_workspace_bytes(M, N, K) the full
 *     split is used; with less, as many slices as fit (fewer than two: the
 *     plain mxfp8_gemm path, no workspace touched).
 * Argument errors as mxfp8_gemm.  Two kernels on `stream`, no allocation, no
 * synchronization.
 */
mxfp8_status mxfp8_gemm_splitk(const uint8_t *a_q, const uint8_t *a_s,
                               const uint8_t *b_q, const uint8_t *b_s,
                               mxfp8_layout b_layout, int64_t M, int64_t N, int64_t K,
                               void *c, mxfp8_dtype c_dtype, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes mxfp8_gemm_splitk uses for this shape on the current
 * device (0: it would not split; also 0 for invalid shapes or no device). */
size_t mxfp8_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * mxfp8_gemm_packed_splitk -- mxfp8_gemm_packed for shapes with few output
 * tiles (small M: section "Speed: when it pays off", as mxfp8_gemm_splitk).
 *
 * Same operands, result and error bound as mxfp8_gemm_packed (A and B in the
 * mxfp8_repack layout, K % 128 == 0), split as mxfp8_gemm_splitk splits: the
 * same slices (sized by mxfp8_gemm_splitk_workspace_bytes(M, N, K); with a
 * smaller workspace, as many slices as fit), the fp32 partial tiles in
 * `workspace`, summed in slice order.  C is bit-identical to
 * mxfp8_gemm_splitk over the canonical grids of the same operands (the same
 * per-slice products in the same order).  workspace: DEVICE memory owned by
 * the caller, 16-byte aligned, or NULL; contents on entry ignored, on return
 * unspecified.  No split (too many tiles, fewer than two slices fit,
 * N % 4 != 0, or mxfp8_gemm_packed would take its 128-row tiles, those fill
 * at least half the compute units and K is at most 64 x 128, where the unsplit
 * launch is the faster): the plain mxfp8_gemm_packed path, no workspace
 * touched.
 * Argument errors as mxfp8_gemm_packed, plus MXFP8_ERR_ALIGN for a workspace
 * not 16-byte aligned.  Two kernels on `stream`, no allocation, no
 * synchronization.
 */
mxfp8_status mxfp8_gemm_packed_splitk(const uint8_t *a_q_packed, const uint8_t *a_s_packed,
                                      const uint8_t *b_q_packed, const uint8_t *b_s_packed,
                                      int64_t M, int64_t N, int64_t K, void *c, mxfp8_dtype c_dtype,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp8_gemm_splitk_noalloc -- mxfp8_gemm_splitk with no caller workspace and
 * no allocation, for callers that cannot allocate device memory (code under
 * HIP-graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operands, result, error bound and launches as mxfp8_gemm_splitk given
 * a workspace of mxfp8_gemm_splitk_workspace_bytes(M, N, K) bytes (the same
 * bits); the fp32 partial tiles go to a static device array inside the
 * library of 32 MiB + 4 KiB per device (held by every device the library
 * runs on until the process ends; every split plan on a 256-CU device fits
 * it).  A plan that would need more returns MXFP8_ERR_SHAPE and enqueues
 * nothing; a shape that does not split runs mxfp8_gemm and touches no
 * scratch.  The array is shared by every call on a device and keeps the last
 * call's partials: calls that overlap on one device (different streams or
 * threads) race on it and must be serialized by the caller.  No allocation,
 * no memset, no synchronization; the first call on a device looks up the
 * array's device address (hipGetSymbolAddress) once.
 */
mxfp8_status mxfp8_gemm_splitk_noalloc(const uint8_t *a_q, const uint8_t *a_s,
                                       const uint8_t *b_q, const uint8_t *b_s,
                                       mxfp8_layout b_layout, int64_t M, int64_t N, int64_t K,
                                       void *c, mxfp8_dtype c_dtype, hipStream_t stream);

/*
 * mxfp8_grouped_gemm -- MoE expert GEMM over groups of rows:
 *   for g in 0..G-1:  C[o_g : o_{g+1}] = A[o_g : o_{g+1}] * B_g^T
 *
 * The page's MoE serving path runs its expert GEMMs in MXFP8 from weights
 * stored in a kernel-specific order (section "The pipeline", sampler
 * paragraph; section "Speed: when it pays off": expert GEMMs dominate MoE
 * decode and FP8 halves their weight traffic).
 *
 *   A               : canonical MXFP8 q[M_total][K], s[M_total][K/32]; rows
 *                     sorted by expert, each group padded to a multiple of 32.
 *   B               : mxfp8_repack output for batch = G matrices [N][K].
 *   d_group_offsets : DEVICE int32 [G+1], non-decreasing, o_0 >= 0,
 *                     o_G <= M_total, every o_g % 32 == 0.  Read on the
 *                     device (no host synchronization); offsets violating
 *                     this are clamped to [0, M_total] and empty groups
 *                     are skipped, never read out of bounds.
 *   C               : [M_total][N]; rows outside [o_0, o_G) are not written.
 * G >= 1, M_total >= 0 (0 enqueues nothing), M_total % 32 == 0, N >= 1,
 * K >= 32, K % 32 == 0.
 */
mxfp8_status mxfp8_grouped_gemm(const uint8_t *a_q, const uint8_t *a_s,
                                const uint8_t *b_q_packed,
                                const uint8_t *b_s_packed,
                                const int32_t *d_group_offsets, int64_t G,
                                int64_t M_total, int64_t N, int64_t K, void *c,
                                mxfp8_dtype c_dtype, hipStream_t stream);

/*
 * mxfp8_grouped_gemm_packed -- mxfp8_grouped_gemm with A in the packed layout.
 *
 * The expert GEMMs' token rows quantized straight into the kernel layout
 * (mxfp8_quantize_many_layouts, MXFP8_PACKED, or mxfp8_repack of the
 * canonical grid), as the dense mxfp8_gemm_packed reads them (section "The
 * pipeline", sampler paragraph: kernel-specific layouts).
 *   A : the mxfp8_repack layout of q[M_total][K], s[M_total][K/32]
 *       (batch 1, N = M_total; mxfp8_packed_bytes(1, M_total, K, 0 / 1)).
 *   B, d_group_offsets, C, G, M_total, N: as mxfp8_grouped_gemm.
 * K % 128 == 0 (MXFP8_ERR_SHAPE otherwise).  C is bit-identical to
 * mxfp8_grouped_gemm over the canonical grid of the same A (the same products
 * in the same order per element); rows outside [o_0, o_G) are not written.
 * Each tile's A copies read 8-row segments of its panel rows, so a group
 * starting inside a panel costs nothing extra; segments past the group's
 * rows read zeros, never the next group's rows.  No allocation, no
 * synchronization.
 */
mxfp8_status mxfp8_grouped_gemm_packed(const uint8_t *a_q_packed, const uint8_t *a_s_packed,
                                       const uint8_t *b_q_packed, const uint8_t *b_s_packed,
                                       const int32_t *d_group_offsets, int64_t G, int64_t M_total,
                                       int64_t N, int64_t K, void *c, mxfp8_dtype c_dtype,
                                       hipStream_t stream);

/*
 * mxfp8_grouped_gemm_wgrad -- the experts' weight gradients:
 *   for g in 0..G-1:  C[g] = A[:, o_g : o_{g+1}] * B[:, o_g : o_{g+1}]^T
 *
 * The weight-gradient GEMM reduces over tokens, so its operands are blocked
 * along the token dimension ("The pipeline", learner paragraph); for an
 * expert the reduction runs over that expert's (padded) token group only.
 * With the token rows sorted by expert, dY^T and X^T quantized along tokens
 * (mxfp8_quantize axis 0 of dY [T][M] and X [T][N]) hold every group's block
 * columns contiguously, and expert g's gradient dW_g = dY_g^T X_g is this
 * GEMM over columns [o_g, o_{g+1}):
 *   A (a_q, a_s): [M][T] / [M][T/32] (axis-0 quantize output of dY [T][M]);
 *   B (b_q, b_s): [N][T] / [N][T/32] (axis-0 quantize output of X [T][N]);
 *   d_group_offsets: DEVICE int32 [G+1] token offsets, non-decreasing,
 *     multiples of 32 (clamped into [0, T]; a malformed table can only drop
 *     work, never address outside the operands);
 *   C: [G][M][N], FP32 or BF16; an empty group's C[g] is all zeros.
 * T % 32 == 0, 32 <= T < 2^23, M, N >= 1, G <= 65535.  Same accumulation and
 * error bound as mxfp8_gemm.  Deterministic.
 * Speed: with T % 128 == 0, a group whose range starts and ends on a multiple
 * of 128 runs the aligned path (scale bytes copied as dwords with the tiles);
 * other groups read scale bytes one per lane, several times slower.
 * mxfp8_quantize_dual_grouped writes the operands in such a layout.
 */
mxfp8_status mxfp8_grouped_gemm_wgrad(const uint8_t *a_q, const uint8_t *a_s,
                                      const uint8_t *b_q, const uint8_t *b_s,
                                      const int32_t *d_group_offsets, int64_t G, int64_t T,
                                      int64_t M, int64_t N, void *c, mxfp8_dtype c_dtype,
                                      hipStream_t stream);

/*
 * mxfp8_grouped_gemm_wgrad_packed -- mxfp8_grouped_gemm_wgrad with both
 * operands in the GEMM's packed layout along the token axis.
 *
 *   A (a_q_packed, a_s_packed): the packed layout of [M][T] (N = M, K = T;
 *     mxfp8_packed_bytes(1, M, T, 0 / 1) bytes);
 *   B (b_q_packed, b_s_packed): the packed layout of [N][T];
 *   d_group_offsets: DEVICE int32 [G+1] token offsets; expert g reduces over
 *     the k-steps [o_g / 128, ceil(o_{g+1} / 128)) of the token axis, so
 *     well-formed tables hold multiples of 128 (as
 *     mxfp8_quantize_dual_grouped_packed's regrouped grid); offsets are
 *     clamped into [0, T], so a malformed table can only give wrong sums,
 *     never address outside the operands;
 *   C: [G][M][N], FP32 or BF16; an empty group's C[g] is all zeros.
 * T % 32 == 0, N % 4 == 0 (FP32) or N % 8 == 0 (BF16), the limits of
 * mxfp8_repack for both operands, G <= 65535.  For 128-aligned groups C is
 * bit-identical to mxfp8_grouped_gemm_wgrad over the canonical grids (same
 * products, same order).  Deterministic; no allocation, no synchronization.
 * Speed: on the Qwen3-30B-A3B learner's weight gradients this launch is
 * slower than mxfp8_grouped_gemm_wgrad's aligned path (its 256x128 tiles
 * copy more operand bytes per output than the aligned path's 256x256 ones,
 * and four of its eight waves store each tile's FP32 C); it serves callers
 * that keep one layout.
 */
mxfp8_status mxfp8_grouped_gemm_wgrad_packed(const uint8_t *a_q_packed, const uint8_t *a_s_packed,
                                             const uint8_t *b_q_packed, const uint8_t *b_s_packed,
                                             const int32_t *d_group_offsets, int64_t G, int64_t T, int64_t M,
                                             int64_t N, void *c, mxfp8_dtype c_dtype, hipStream_t stream);

/*
 * mxfp8_selfcheck -- post-sync check of one quantized layer's serving path.
 *
 * The page's post-sync self-check (section "Correctness: how it fails",
 * run-time check C3): after every synchronization one quantized layer runs
 * through the serving kernel on random input and is compared with a
 * high-precision GEMM on the dequantized synchronized weights; healthy layers
 * are a few percent off (about 0.027 dense, 0.049 expert on the page), stale
 * derived layouts are off by order 1, and the page's tolerance is 0.25.
 *
 *   Y     = mxfp8_gemm(quantize(x, axis 1), packed weights)      (fp32 out)
 *   Y_ref = x * W'^T in fp32, W' = dequantize(w_q, w_s)           (canonical)
 *   d_result[0] = ||Y - Y_ref||_F / ||Y_ref||_F, d_result[1] = ||Y - Y_ref||^2,
 *   d_result[2] = ||Y_ref||^2 (fp64); d_result[0] is NaN if either output is
 *   not finite or Y_ref is zero.
 *
 * x: BF16 probe [M][K] (device; the caller draws it, e.g. N(0,1)), M <= 4096.
 * w_q / w_s: the synchronized canonical grid [N][K], [N][K/32].
 * w_q_packed / w_s_packed: the storage the serving GEMM reads (mxfp8_repack
 *   layout, one matrix; for expert g of a batch pass the g-th matrix's
 *   offsets, g * mxfp8_packed_bytes(1, N, K, which)).
 * workspace: device, mxfp8_selfcheck_workspace_bytes(M, N, K) bytes, 16-byte
 *   aligned, owned by the caller.  d_result: device, 3 doubles.
 * Asynchronous like every call here: the verdict is read after the stream is
 * synchronized (the Python binding applies the tolerance and the off / warn
 * / error mode).  Deterministic.
 */
size_t mxfp8_selfcheck_workspace_bytes(int64_t M, int64_t N, int64_t K);

mxfp8_status mxfp8_selfcheck(const void *x_bf16, int64_t M, int64_t N, int64_t K,
                             const uint8_t *w_q, const uint8_t *w_s,
                             const uint8_t *w_q_packed, const uint8_t *w_s_packed,
                             void *workspace, double *d_result, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *mxfp8_status_string(mxfp8_status status);

/* The HIP error code of the calling thread's last MXFP8_ERR_HIP (0 if none). */
int mxfp8_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char *mxfp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
