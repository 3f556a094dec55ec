// device_common.hpp -- gfx950 device helpers shared by the NVFP4 kernels.
//
// Everything here is written for CDNA4 (wave64, BF16 MFMA, OCP FP8/FP4
// conversion instructions).  No other target is supported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;

// Largest finite E4M3 (OCP FN) value and the E2M1 maximum; the tensor-level
// divisor is their product.
constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

// ---- encoders (round to nearest, ties to even, saturating) ----------------

// E4M3 (OCP FN) code of a non-negative finite float; sign bit 0.
// Normal range (x >= 2^-6): round the float's mantissa to 3 bits by adding
// the half-ulp bias plus the parity of the kept LSB, then rebias the exponent
// from 127 to 7.  Subnormal range: the code is rint(x * 2^9) (exact scaling,
// ties to even); a result of 8 is the smallest normal code, as it should be.
__device__ __forceinline__ uint32_t encode_e4m3(float x) {
  if (x >= kE4M3Max) return 0x7Eu;
  if (x < 0.015625f) {  // 2^-6
    return (uint32_t)__builtin_rintf(x * 512.0f);
  }
  uint32_t u = __float_as_uint(x);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;  // 8-bit exponent | 3-bit mantissa
  uint32_t code = r - ((127u - 7u) << 3);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Correctly rounded FP32 quotient |x| / d for the element encoder (d > 0).
// Where d lies in [2^-98, 2^100] (`fast`), it is formed from the correctly
// rounded reciprocal r = RN(1/d) with one FMA-based correction (Markstein's
// method: q0 = RN(|x| r), e = |x| - q0 d exactly, q = RN(q0 + e r), which is
// RN(|x| / d) for normal operands); otherwise, and for d == 0 (quotient 0),
// the IEEE division is used.
__device__ __forceinline__ bool element_divisor(float d, float& r) {
  const bool fast = d >= 0x1p-98f && d <= 0x1p100f;
  r = fast ? 1.0f / d : 0.0f;  // IEEE division: correctly rounded
  return fast;
}
__device__ __forceinline__ float element_quotient(float x, float d, float r, bool fast) {
  const float ax = __builtin_fabsf(x);
  if (fast) {
    const float q0 = ax * r;
    return __builtin_fmaf(__builtin_fmaf(-q0, d, ax), r, q0);
  }
  return d != 0.0f ? ax / d : 0.0f;
}

// Two E2M1 codes into nibbles 2 SEL and 2 SEL + 1 of `word`: gfx950's FP32 ->
// FP4 pack conversion with scale operand 1.0 gives the sign bit of each input
// followed by its nearest E2M1 magnitude, ties to the even code (0.25 -> 0,
// 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4), saturating at
// 6; the sign is kept on a zero magnitude.
template <int SEL>
__device__ __forceinline__ uint32_t pack_e2m1_pair(uint32_t word, float q0, float q1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, SEL);
}

// ---- decoders ---------------------------------------------------------------

// E4M3 byte `sel` (0..3) of a dword to float (gfx950 converts OCP E4M3FN).
template <int sel>
__device__ __forceinline__ float decode_e4m3(uint32_t dword) {
  return __builtin_amdgcn_cvt_f32_fp8(dword, sel);
}

// Eight E2M1 nibbles (one dword, element 2j in the low nibble of byte j) times
// a block scale, as eight BF16 values in k order.  The scaled conversion
// instruction applies only the exponent of its scale operand, so it is run with
// scale 1.0 and the exact product e2m1 * scale is formed in FP32; its upper 16
// bits are the BF16 value (the product has at most 6 significant bits).
__device__ __forceinline__ bf16x8_t dequant8(uint32_t nib, float scale) {
  u32x4_t out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    f32x2_t v;
    switch (p) {
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 3); break;
    }
    float lo = v.x * scale;
    float hi = v.y * scale;
    out[p] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  bf16x8_t r;
  __builtin_memcpy(&r, &out, sizeof(r));
  return r;
}

// Round-to-nearest-even FP32 -> BF16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- memory ordering for split-K hand-off -----------------------------------

__device__ __forceinline__ void fence_release_agent() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void fence_acquire_agent() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

}  // namespace nvfp4
