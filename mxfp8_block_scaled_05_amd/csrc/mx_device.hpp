// Device-side building blocks shared by the gfx950 MXFP8 kernels.
//
// Written for CDNA4 (gfx950) only: 64-wide wavefronts, OCP E4M3 conversion
// instructions, scaled MFMA, buffer loads straight into LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over [base, base + bytes): out-of-range lanes read 0 and
// never touch memory.  Data format field = 32-bit, as gfx9 buffers expect.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Offset that is always outside any buffer this library builds (bytes <
// 2^31), so the lane reads zero.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ float bits_to_float(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t float_to_bits(float f) { return __float_as_uint(f); }

// 2^(127 - code) as an fp32 (normal for code in [0, 246]); multiplying a
// BF16 value by it is exact (or underflows far below E4M3's smallest
// subnormal, where the result rounds to a signed zero either way).
__device__ __forceinline__ float inv_scale_from_code(uint32_t code) {
    return bits_to_float((254u - code) << 23);
}

// Scale code from the BF16 exponent field of the block's max magnitude:
//   finite amax with field E >= 1 : floor(log2 amax) = E - 127, s = E - 135,
//                                    code = max(s, -127) + 127 = max(E - 8, 0)
//   zero or subnormal amax        : code 0 (s clamped to -127)
//   Inf / NaN (E = 255)           : code 0xFF
__device__ __forceinline__ uint32_t scale_code_from_amax_bits(uint32_t amax_mag_bits) {
    uint32_t e = amax_mag_bits >> 7;      // BF16 magnitude 0x0000..0x7FFF -> field 0..255
    uint32_t code = e > 8u ? e - 8u : 0u;
    return e == 255u ? 255u : code;
}

// Two scaled values -> two E4M3 bytes in the selected 16-bit half of `old`.
// The hardware conversion rounds to nearest even; values are clamped to
// +-448 first, which is exactly the saturating rule (|v| >= 448 -> 0x7E).
template <bool HI>
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old) {
    a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
    b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

typedef float v2f __attribute__((ext_vector_type(2)));

// Two fp32 -> two BF16 (a in bits 0-15, b in bits 16-31) with gfx950's packed
// conversion: round to nearest even, a NaN stays a quiet NaN with its sign and
// upper payload.  Checked on MI355X against the integer rounding
// (u + 0x7FFF + ((u >> 16) & 1)) >> 16 with NaN -> (u >> 16) | 0x40: equal on
// every upper half combined with six lower halves (0, 1, 0x7FFF, 0x8000,
// 0x8001, 0xFFFF) and on 2^20 random words.  One instruction per pair, where
// the integer form took about fifteen per value.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return bf16x2_rne(f, 0.0f) & 0xFFFFu; }

// XOR swizzle of the 16-byte chunk slots inside a 128-byte LDS row: chunk c
// of row r sits at slot c ^ (r % 8).  Measured on gfx950 with the LDS
// counters (ds_read_b128, each group of 16 lanes reading 16 consecutive rows
// at one chunk): this spreads the reads over the banks as a linear read does,
// while the variant c ^ ((r % 8) ^ (r / 8 % 2)) takes twice the LDS cycles
// per read (half of them bank-conflict stalls).
__device__ __forceinline__ uint32_t swz(uint32_t row) { return row & 7u; }

}  // namespace mx
