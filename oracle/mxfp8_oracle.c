/*
 * MXFP8 oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of what the MXFP8 hot path computes.
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this file's library.  The HIP library never links or calls it, and
 * this file includes nothing from the library (it shares no header, table or
 * helper with it).
 *
 * What it follows:
 *  - "End-to-End MXFP8 RL on Blackwell: What Matching Buys, When It Pays Off,
 *    and How It Fails" (verl blog), section "The pipeline", paragraph "The
 *    format": along the summed axis, every 32 consecutive values become 32
 *    E4M3 codes and one E8M0 power-of-two scale byte (8 + 8/32 bits each).
 *  - same page, section "The pipeline", paragraph on the learner: the
 *    weight-gradient GEMM reduces over tokens, so some operands are blocked
 *    in 32s along the token dimension (axis 0 here).
 *  - same page, section "Correctness: how it fails", "Post-sync self-check":
 *    the reference for the MXFP8 GEMM is a high-precision GEMM on the
 *    dequantized operands.
 *  - the OCP Microscaling Formats (MX) v1.0 specification that the format
 *    paragraph cites: E4M3 ("FN": bias 7, max 448, NaN = S.1111.111, no Inf),
 *    E8M0 (2^(c-127), 0xFF = NaN), shared exponent
 *    floor(log2(max|x|)) - emax_elem with emax_elem = 8 for E4M3, elements
 *    rounded to nearest-even and clamped to +-448.
 *
 * Readings where the pages are silent (all zero block -> scale code 0, any
 * NaN/Inf in a block -> scale 0xFF and elements 0x7F, no flush of BF16
 * subnormals, scale exponent clamped to >= -127) are stated at each function.
 *
 * Arithmetic is fp64; every product of an E4M3 value with a power of two and
 * every E4M3 x E4M3 product used here is exact in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MXO_BLOCK 32

/* ---------------------------------------------------------------- codecs */

/* BF16 bit pattern -> its real value (exact in fp64; subnormals kept). */
double mxo_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Real value -> nearest BF16, ties to even (IEEE roundTiesToEven).  Written
 * from the definition: find the value's binade, its quantum, round the
 * quotient to an integer with rint() (ties to even in the default mode).  */
uint16_t mxo_bf16_encode(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                /* floor(log2 a)              */
    if (e < -126) e = -126;                 /* subnormal range shares 2^-126's quantum */
    double quantum = ldexp(1.0, e - 7);     /* 7 stored mantissa bits */
    double n = rint(a / quantum);           /* exact division by a power of two */
    double r = n * quantum;
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;   /* overflow rounds to Inf */
    float rf = (float)r;                     /* exact: r is a BF16 value */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* E4M3 (OCP "FN") code -> value.  S.EEEE.MMM, bias 7:
 *   E = 0      : (-1)^S * (M/8) * 2^-6          (subnormal)
 *   E = 1..15  : (-1)^S * (1 + M/8) * 2^(E-7)
 *   E = 15,M = 7 is NaN; there is no infinity.                          */
double mxo_e4m3_decode(uint8_t c) {
    int s = (c >> 7) & 1, E = (c >> 3) & 0xF, M = c & 7;
    if (E == 15 && M == 7) return NAN;
    double mag = (E == 0) ? ldexp((double)M / 8.0, -6)
                          : ldexp(1.0 + (double)M / 8.0, E - 7);
    return s ? -mag : mag;
}

/* E8M0 code -> 2^(c-127); 0xFF is NaN. */
double mxo_e8m0_decode(uint8_t c) {
    if (c == 0xFF) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* Value -> E4M3 code, round to nearest with ties to even, saturating to
 * +-448 (0x7E/0xFE) at or above the largest finite magnitude.  The sign of
 * zero is kept.  NaN -> 0x7F.                                              */
uint8_t mxo_e4m3_encode(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    e -= 1;                          /* floor(log2 a)                         */
    if (e < -6) e = -6;              /* subnormals share the 2^-6 binade's quantum */
    double quantum = ldexp(1.0, e - 3);   /* 3 mantissa bits */
    int n = (int)rint(a / quantum);       /* 0..16, ties to even */
    if (n == 16) { e += 1; n = 8; }       /* rounded up into the next binade */
    if (n < 8) return sign | (uint8_t)n;  /* subnormal (only when e == -6)   */
    return sign | (uint8_t)(((e + 7) << 3) | (n - 8));
}

/* Element-wise array forms of the two E4M3 conversions (for exhaustive
 * sweeps from the tests; same functions as above, applied per element). */
void mxo_e4m3_encode_n(const double *v, int64_t n, uint8_t *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_e4m3_encode(v[i]);
}

void mxo_e4m3_decode_n(const uint8_t *c, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_e4m3_decode(c[i]);
}

/* ----------------------------------------------------------- block scale */

/* Shared scale code of one 32-element BF16 block (elements x[i*stride]).
 *  - amax = max |x_i| (exact).
 *  - amax finite and > 0: s = floor(log2 amax) - 8, clamped to s >= -127
 *    (E8M0's smallest value); code = s + 127.  BF16 subnormals count with
 *    their true value.
 *  - all-zero block: code 0 (floor(log2 0) = -inf, clamped).
 *  - any NaN or +-Inf in the block: code 0xFF (E8M0 NaN).                  */
uint8_t mxo_block_scale(const uint16_t *x, int64_t stride) {
    double amax = 0.0;
    for (int i = 0; i < MXO_BLOCK; ++i) {
        double v = mxo_bf16_decode(x[(int64_t)i * stride]);
        if (isnan(v) || isinf(v)) return 0xFF;
        if (fabs(v) > amax) amax = fabs(v);
    }
    if (amax == 0.0) return 0;
    int e;
    frexp(amax, &e);
    e -= 1;
    int s = e - 8;
    if (s < -127) s = -127;
    return (uint8_t)(s + 127);
}

/* Quantize one block: scale code, then q_i = encode(x_i * 2^-s). */
static void quantize_block(const uint16_t *x, int64_t stride, uint8_t *q,
                           int64_t qstride, uint8_t *scale_out) {
    uint8_t code = mxo_block_scale(x, stride);
    *scale_out = code;
    for (int i = 0; i < MXO_BLOCK; ++i) {
        if (code == 0xFF) { q[(int64_t)i * qstride] = 0x7F; continue; }
        double v = ldexp(mxo_bf16_decode(x[(int64_t)i * stride]), 127 - (int)code);
        q[(int64_t)i * qstride] = mxo_e4m3_encode(v);
    }
}

/* Quantize a row-major BF16 matrix x[rows][cols].
 *   axis = 1: blocks run along cols (the reduction axis of x as the left
 *             GEMM operand).  q[rows][cols], scales[rows][cols/32].
 *   axis = 0: blocks run along rows (the token axis, for the weight-gradient
 *             operands); the output is written transposed so the block axis
 *             is contiguous: q[cols][rows], scales[cols][rows/32].
 * Returns 0, or -1 if the block axis is not a multiple of 32.            */
int mxo_quantize(const uint16_t *x, int64_t rows, int64_t cols, int axis,
                 uint8_t *q, uint8_t *scales) {
    if (axis == 1) {
        if (cols % MXO_BLOCK) return -1;
        int64_t nb = cols / MXO_BLOCK;
        #pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b)
                quantize_block(x + r * cols + b * MXO_BLOCK, 1,
                               q + r * cols + b * MXO_BLOCK, 1,
                               scales + r * nb + b);
        return 0;
    }
    if (axis == 0) {
        if (rows % MXO_BLOCK) return -1;
        int64_t nb = rows / MXO_BLOCK;
        #pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < cols; ++c)
            for (int64_t b = 0; b < nb; ++b)
                quantize_block(x + b * MXO_BLOCK * cols + c, cols,
                               q + c * rows + b * MXO_BLOCK, 1,
                               scales + c * nb + b);
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------ dequantize */

/* Value of element (r, c) of the original [rows][cols] matrix, from the
 * quantizer's output for the given axis:  decode(q) * 2^(code - 127).     */
static double dq_at(const uint8_t *q, const uint8_t *s, int64_t rows,
                    int64_t cols, int axis, int64_t r, int64_t c) {
    if (axis == 1)
        return mxo_e4m3_decode(q[r * cols + c]) *
               mxo_e8m0_decode(s[r * (cols / MXO_BLOCK) + c / MXO_BLOCK]);
    return mxo_e4m3_decode(q[c * rows + r]) *
           mxo_e8m0_decode(s[c * (rows / MXO_BLOCK) + r / MXO_BLOCK]);
}

void mxo_dequantize_f64(const uint8_t *q, const uint8_t *s, int64_t rows,
                        int64_t cols, int axis, double *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = dq_at(q, s, rows, cols, axis, r, c);
}

/* fp64 -> fp32 by C's conversion (round to nearest even; overflow -> Inf). */
void mxo_dequantize_f32(const uint8_t *q, const uint8_t *s, int64_t rows,
                        int64_t cols, int axis, float *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = (float)dq_at(q, s, rows, cols, axis, r, c);
}

void mxo_dequantize_bf16(const uint8_t *q, const uint8_t *s, int64_t rows,
                         int64_t cols, int axis, uint16_t *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = mxo_bf16_encode(dq_at(q, s, rows, cols, axis, r, c));
}

/* ------------------------------------------------------------------ GEMM */

/* Dequantize rows [r0, r0+nr) of a K-contiguous operand (axis-1 layout:
 * q[rows][K], s[rows][K/32]) into fp64.                                    */
static void dq_rows(const uint8_t *q, const uint8_t *s, int64_t K,
                    const int64_t *row_idx, int64_t nr, double *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nr; ++i) {
        int64_t r = row_idx ? row_idx[i] : i;
        for (int64_t k = 0; k < K; ++k)
            out[i * K + k] = mxo_e4m3_decode(q[r * K + k]) *
                             mxo_e8m0_decode(s[r * (K / MXO_BLOCK) + k / MXO_BLOCK]);
    }
}

/* C_ref[i][n] = sum_k A'[m_i][k] * B'[n][k] and S[i][n] = sum_k |A'[m_i][k] *
 * B'[n][k]| over the dequantized operands, k ascending, fp64.  A is [M][K]
 * and B is [N][K], both K-contiguous (quantizer axis-1 layout, or axis-0
 * output which is already transposed).  Only the requested rows of A are
 * evaluated (all rows when row_idx is NULL and nrows == M).               */
int mxo_gemm_rows(const uint8_t *a_q, const uint8_t *a_s, const uint8_t *b_q,
                  const uint8_t *b_s, int64_t M, int64_t N, int64_t K,
                  const int64_t *row_idx, int64_t nrows, double *c_ref,
                  double *c_abs) {
    (void)M;
    if (K % MXO_BLOCK) return -1;
    double *A = (double *)malloc(sizeof(double) * (size_t)(nrows * K + 1));
    double *B = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!A || !B) { free(A); free(B); return -2; }
    dq_rows(a_q, a_s, K, row_idx, nrows, A);
    dq_rows(b_q, b_s, K, NULL, N, B);
    #pragma omp parallel for schedule(static) collapse(2)
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = A[i * K + k] * B[n * K + k];
                acc += p;
                mag += fabs(p);
            }
            c_ref[i * N + n] = acc;
            if (c_abs) c_abs[i * N + n] = mag;
        }
    free(A);
    free(B);
    return 0;
}

/* Grouped GEMM: rows [off[g], off[g+1]) of A multiply expert g's weight
 * B_g[N][K] (B = G stacked [N][K] matrices, canonical layout).  For each
 * requested row m the expert is the g with off[g] <= m < off[g+1]; a row in
 * no group is left untouched and flagged by -1 in grp_out.               */
int mxo_grouped_gemm_rows(const uint8_t *a_q, const uint8_t *a_s,
                          const uint8_t *b_q, const uint8_t *b_s,
                          const int32_t *off, int64_t G, int64_t M_total,
                          int64_t N, int64_t K, const int64_t *row_idx,
                          int64_t nrows, double *c_ref, double *c_abs,
                          int32_t *grp_out) {
    if (K % MXO_BLOCK) return -1;
    int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nrows + 1));
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nrows + 1));
    double *cr = (double *)malloc(sizeof(double) * (size_t)(nrows * N + 1));
    double *ca = (double *)malloc(sizeof(double) * (size_t)(nrows * N + 1));
    if (!sel || !pos || !cr || !ca) { free(sel); free(pos); free(cr); free(ca); return -2; }
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t m = row_idx ? row_idx[i] : i;
        int32_t g = -1;
        for (int64_t j = 0; j < G; ++j)
            if (off[j] <= m && m < off[j + 1]) { g = (int32_t)j; break; }
        if (grp_out) grp_out[i] = g;
    }
    int rc = 0;
    for (int64_t g = 0; g < G && rc == 0; ++g) {
        int64_t n_sel = 0;
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t m = row_idx ? row_idx[i] : i;
            if (off[g] <= m && m < off[g + 1]) { sel[n_sel] = m; pos[n_sel] = i; ++n_sel; }
        }
        if (!n_sel) continue;
        rc = mxo_gemm_rows(a_q, a_s, b_q + g * N * K, b_s + g * N * (K / MXO_BLOCK),
                           M_total, N, K, sel, n_sel, cr, ca);
        for (int64_t t = 0; t < n_sel && rc == 0; ++t) {
            memcpy(c_ref + pos[t] * N, cr + t * N, sizeof(double) * (size_t)N);
            if (c_abs) memcpy(c_abs + pos[t] * N, ca + t * N, sizeof(double) * (size_t)N);
        }
    }
    free(sel); free(pos); free(cr); free(ca);
    return rc;
}

/* ---------------------------------------------------- packed weight layout
 *
 * The packed ("kernel") layout of a batch of canonical weights q[b][N][K],
 * s[b][N][K/32], written here from its specification (the library's public
 * header states the same specification in words):
 *
 *   panels of 256 rows (NP = ceil(N/256)), k-steps of 128 (KS = ceil(K/128)).
 *   elements: [b][panel][kstep][row 0..255][128 bytes]; inside a row the
 *     16-byte chunk c (k = kstep*128 + 16c .. +15) sits at chunk position
 *     c ^ (row % 8).  Rows >= N and k >= K are 0.
 *   scales: [b][panel][kstep][atom 0..15 of 16 rows][lane 0..63] bytes; byte
 *     (panel, kstep, atom, lane) is the scale of row 256*panel + 16*atom +
 *     (lane % 16), block 4*kstep + (lane / 16).  Rows >= N or blocks >= K/32
 *     hold 127 (the code of 1.0).
 */
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t mxo_packed_bytes(int64_t batch, int64_t N, int64_t K, int which) {
    int64_t NP = ceil_div(N, 256), KS = ceil_div(K, 128);
    if (which == 0) return batch * NP * KS * 256 * 128;
    return batch * NP * KS * 16 * 64;
}

static int64_t pk_elem_offset(int64_t N, int64_t K, int64_t b, int64_t n, int64_t k) {
    int64_t NP = ceil_div(N, 256), KS = ceil_div(K, 128);
    int64_t panel = n / 256, row = n % 256, ks = k / 128, kin = k % 128;
    int64_t c = kin / 16, f = row % 8;
    return (((b * NP + panel) * KS + ks) * 256 + row) * 128 + ((c ^ f) * 16) + kin % 16;
}

static int64_t pk_scale_offset(int64_t N, int64_t K, int64_t b, int64_t n, int64_t blk) {
    int64_t NP = ceil_div(N, 256), KS = ceil_div(K, 128);
    int64_t panel = n / 256, atom = (n % 256) / 16, lane = (n % 16) + 16 * (blk % 4);
    int64_t ks = blk / 4;
    return (((b * NP + panel) * KS + ks) * 16 + atom) * 64 + lane;
}

/* canonical -> packed (padding written as specified) */
int mxo_pack(const uint8_t *q, const uint8_t *s, int64_t batch, int64_t N,
             int64_t K, uint8_t *qp, uint8_t *sp) {
    if (K % MXO_BLOCK || N <= 0 || K <= 0 || batch < 0) return -1;
    memset(qp, 0, (size_t)mxo_packed_bytes(batch, N, K, 0));
    memset(sp, 127, (size_t)mxo_packed_bytes(batch, N, K, 1));
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                qp[pk_elem_offset(N, K, b, n, k)] = q[(b * N + n) * K + k];
            for (int64_t blk = 0; blk < K / MXO_BLOCK; ++blk)
                sp[pk_scale_offset(N, K, b, n, blk)] = s[(b * N + n) * (K / MXO_BLOCK) + blk];
        }
    return 0;
}

/* packed -> canonical (the inverse; padding is ignored) */
int mxo_unpack(const uint8_t *qp, const uint8_t *sp, int64_t batch, int64_t N,
               int64_t K, uint8_t *q, uint8_t *s) {
    if (K % MXO_BLOCK || N <= 0 || K <= 0 || batch < 0) return -1;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                q[(b * N + n) * K + k] = qp[pk_elem_offset(N, K, b, n, k)];
            for (int64_t blk = 0; blk < K / MXO_BLOCK; ++blk)
                s[(b * N + n) * (K / MXO_BLOCK) + blk] = sp[pk_scale_offset(N, K, b, n, blk)];
        }
    return 0;
}
