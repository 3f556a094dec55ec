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

// Direct global -> LDS loads (buffer_load ... lds): lane l writes its bytes
// at M0 + l * size.  They are issued from inline assembly so that the
// compiler does not treat every later LDS read as a possible alias of an
// in-flight load and wait for all of them (which would serialize a ring of
// stages); the kernels wait for exactly the loads they need with explicit
// vmcnt waits.  M0 is saved and restored around each load.
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32), bytes, 0x00020000u};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)(p);
}

// COH: a device-coherent load (sc1), for data another XCD wrote during the
// same launch (which this XCD's L2 may hold stale).
template <bool COH = false>
__device__ __forceinline__ void lds_dma16(uint32_t lds, uint32_t voff, uint32_t soff,
                                          u32x4_t rsrc) {
  // the descriptor is uniform; say so, so that it stays in SGPRs
  rsrc = u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane(rsrc[0]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[1]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[2]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[3])};
  uint32_t saved;
  if constexpr (COH)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen sc1 lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
          "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
          "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
}

// s_waitcnt vmcnt(n) for a run-time n: the immediate must be a constant.
// Encoding (gfx9): vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt
// and lgkmcnt left at their maxima (no wait on them).  n >= 63 needs no
// wait (the counter cannot exceed 63); n <= 0 waits for everything.
__device__ __forceinline__ void wait_vmcnt(int n) {
#define NVFP4_VMCNT(v) \
  case v: __builtin_amdgcn_s_waitcnt(((v) & 15) | (((v) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
#define NVFP4_VMCNT8(b) NVFP4_VMCNT(b) NVFP4_VMCNT(b + 1) NVFP4_VMCNT(b + 2) NVFP4_VMCNT(b + 3) \
  NVFP4_VMCNT(b + 4) NVFP4_VMCNT(b + 5) NVFP4_VMCNT(b + 6) NVFP4_VMCNT(b + 7)
  if (n >= 63) return;
  switch (n) {
    NVFP4_VMCNT8(8) NVFP4_VMCNT8(16) NVFP4_VMCNT8(24) NVFP4_VMCNT8(32) NVFP4_VMCNT8(40)
    NVFP4_VMCNT8(48) NVFP4_VMCNT(1) NVFP4_VMCNT(2) NVFP4_VMCNT(3) NVFP4_VMCNT(4)
    NVFP4_VMCNT(5) NVFP4_VMCNT(6) NVFP4_VMCNT(7) NVFP4_VMCNT(56) NVFP4_VMCNT(57)
    NVFP4_VMCNT(58) NVFP4_VMCNT(59) NVFP4_VMCNT(60) NVFP4_VMCNT(61) NVFP4_VMCNT(62)
    default: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); break;
  }
#undef NVFP4_VMCNT8
#undef NVFP4_VMCNT
}

// s_waitcnt lgkmcnt(0): this wave's LDS (and scalar) accesses have completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N < 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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
