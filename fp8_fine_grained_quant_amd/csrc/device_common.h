// device_common.h -- small gfx950 device helpers shared by the quantize and
// GEMM kernels of libfp8q.  Internal header; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace fp8q {

// Largest finite OCP E4M3 magnitude: 1.75 * 2^8.
constexpr float kE4M3Max = 448.0f;
constexpr float kFltMax = 3.402823466e+38f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two FP32 values to a packed BF16 pair (lo in bits 0-15), rounded to
// nearest even: one v_cvt_pk_bf16_f32, under the wave's default FP32 mode
// (round to nearest even, denormals kept).  Same bits as the integer
// rounding u + 0x7FFF + ((u >> 16) & 1) on finite inputs (the GEMM tests pin
// ties, subnormals and underflow to zero), in one instruction instead of ~7.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Max over the 16 lanes of a DPP row, on non-negative FP32 values compared
// as unsigned integers (their bit patterns order like the values).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));  // row_ror:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));  // row_ror:1
    return v;
}

// Group scale rule: s = amax/448 (dequantization factor) and
// inv = min(448/amax, FLT_MAX), both correctly rounded FP32 divisions
// (amax == 0 gives 448/0 = +inf, clamped to FLT_MAX).
__device__ __forceinline__ void group_scale(float amax, float& s, float& inv) {
    s = amax / kE4M3Max;
    inv = fminf(kE4M3Max / amax, kFltMax);
}

// Power-of-two rule (the value an E8M0 exponent carries): s = 2^e with e the
// smallest integer such that amax <= 448 * 2^e, clamped to [-127, 127], and
// inv = 2^-e.  For a normal amax = 1.f * 2^k, 448 * 2^e = 1.75 * 2^(8+e), so
// e = k - 8 when 1.f <= 1.75 (mantissa field <= 0x600000) and k - 7 above;
// zero and subnormal amax (k <= -127) clamp to e = -127.  s = 2^-127 is the
// FP32 subnormal 0x00400000; inv's exponent field 127 - e stays in [6, 254].
__device__ __forceinline__ void group_scale_pow2(float amax, float& s, float& inv) {
    const uint32_t b = __float_as_uint(amax);
    int e = -127;
    if (b >= 0x00800000u) {
        const int k = (int)(b >> 23) - 127;
        e = max(k - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0), -127);
    }
    s = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
    inv = __uint_as_float((uint32_t)(127 - e) << 23);
}

template <int RULE>
__device__ __forceinline__ void group_scale_rule(float amax, float& s, float& inv) {
    if (RULE == kRulePow2) group_scale_pow2(amax, s, inv);
    else group_scale(amax, s, inv);
}

// Encode 4 FP32 values (already multiplied by inv) into one dword, byte i =
// code of v_i.  Each value is clamped to +-448 first (saturation), then
// converted by the hardware's round-to-nearest-even FP32 -> OCP E4M3
// conversion, two values per instruction into one 16-bit half.
__device__ __forceinline__ uint32_t enc4(float v0, float v1, float v2, float v3) {
    v0 = __builtin_amdgcn_fmed3f(v0, -kE4M3Max, kE4M3Max);
    v1 = __builtin_amdgcn_fmed3f(v1, -kE4M3Max, kE4M3Max);
    v2 = __builtin_amdgcn_fmed3f(v2, -kE4M3Max, kE4M3Max);
    v3 = __builtin_amdgcn_fmed3f(v3, -kE4M3Max, kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
    return (uint32_t)w;
}

}  // namespace fp8q
