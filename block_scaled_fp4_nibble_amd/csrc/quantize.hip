// quantize.hip -- NVFP4 encoding of BF16 weight tensors on gfx950.
//
// Two-tier scaling: one FP32 global scale per tensor plus one FP8-E4M3 scale
// per 16 consecutive values along K ("The Blackwell Architectural Split:
// NVFP4, Attention, and Consumer Silicon", section "Preserving precision --
// dual-tier scale handling"; the A4Q section of the same page works on such
// 16-value blocks).  Global scale g = amax / (6 * 448); block scale =
// E4M3(amax_b / 6 / g); element = E2M1(|w| / (s * g)) with the sign copied.
//
// Pass 1 (amax_partial): each workgroup reduces a slice of one tensor to the
//   largest magnitude, working on BF16 bit patterns (for non-negative IEEE
//   values the integer order is the numeric order, and NaN/Inf patterns sort
//   above every finite one, so one integer max both finds amax and detects
//   non-finite input).  Writes one uint32 per workgroup to the workspace.
// Pass 2 (encode): every workgroup first folds its tensor's partials
//   (deterministic, no atomics), derives g, then its threads encode 16-value
//   blocks in a grid-stride loop: 32 bytes in, 8 packed bytes + 1 scale byte
//   out per block.  The element quotient |w| / d is the correctly rounded
//   FP32 quotient, as in the definition: for d in [2^-98, 2^100] it is formed
//   from the correctly rounded reciprocal r = RN(1/d) with one FMA-based
//   correction (Markstein: q0 = RN(|w| r), e = |w| - q0 d exactly, q =
//   RN(q0 + e r) = RN(|w| / d) for normal operands); an |w| below 2^-100
//   then gives a quotient far below the first rounding threshold (0.25), so
//   its code is 0 either way.  Other blocks use the IEEE division.
// Both passes stream W with 16-byte loads.  Pass 1 reads through the caches,
// so a tensor that fits the 256 MB Infinity Cache is partly read from there
// by pass 2 (8192 x 8192: 66 -> 60 us); pass 2's loads are non-temporal.
#include <algorithm>

#include "device_common.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

constexpr int kQThreads = 256;
constexpr int kQUnroll = 4;  // blocks per thread in flight in the encoder

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

__device__ __forceinline__ uint32_t max_mag_bits(u32x4_t v, uint32_t m) {
  // magnitudes of 8 BF16 values (sign cleared), packed unsigned 16-bit max
  u16x2_t acc;
  __builtin_memcpy(&acc, &m, 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t d = v[i] & 0x7FFF7FFFu;
    u16x2_t dv;
    __builtin_memcpy(&dv, &d, 4);
    acc = __builtin_elementwise_max(acc, dv);
  }
  uint32_t r;
  __builtin_memcpy(&r, &acc, 4);
  return r;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  // wave reduction then across the 4 waves through LDS
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off);
    v = v > o ? v : o;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < kQThreads / kWave; ++i) r = r > red[i] ? r : red[i];
  __syncthreads();
  return r;
}

// grid: (parts, batch).  Tensor t spans elems = n*k BF16 values (a multiple of 16).
__global__ __launch_bounds__(kQThreads) void amax_partial_kernel(
    const uint16_t* __restrict__ w, int64_t elems, uint32_t* __restrict__ partial, int parts) {
  __shared__ uint32_t red[kQThreads / kWave];
  const int t = blockIdx.y;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w + (int64_t)t * elems);
  const int64_t vecs = elems / 8;
  uint32_t m = 0;
  // kQUnroll loads in flight per thread
  const int64_t stride = (int64_t)parts * kQThreads;
  for (int64_t i0 = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i0 < vecs;
       i0 += stride * kQUnroll) {
    u32x4_t v[kQUnroll];
#pragma unroll
    for (int u = 0; u < kQUnroll; ++u)
      v[u] = i0 + u * stride < vecs ? src[i0 + u * stride]
                                    : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kQUnroll; ++u) m = max_mag_bits(v[u], m);
  }
  uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  m = lo > hi ? lo : hi;
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[(int64_t)t * parts + blockIdx.x] = m;
}

// Encode one 16-value block (two 16-byte halves) with global scale g.
__device__ __forceinline__ void encode_block(u32x4_t v0, u32x4_t v1, float g, uint8_t* packed8,
                                             uint8_t* scale1) {
  uint32_t mb = max_mag_bits(v1, max_mag_bits(v0, 0u));
  uint32_t lo = mb & 0xFFFFu, hi = mb >> 16;
  const float amax_b = bf16_bits_to_float(lo > hi ? lo : hi);

  uint32_t scode = 0;
  if (g != 0.0f) {
    const float t6 = amax_b / kE2M1Max;
    scode = encode_e4m3(t6 / g);
  }
  const float s_dec = decode_e4m3<0>(scode);
  const float d = s_dec * g;
  float r;
  const bool fast = element_divisor(d, r);

  // Each pair of elements: the FP32 quotients |w| / d (element_quotient),
  // signed like w, become two E2M1 codes (pack_e2m1_pair); element 2j goes
  // to the low nibble of byte j.  The pack conversion and the quotient are
  // compared with the oracle's definition over every FP32 input pattern and
  // with IEEE division by the GPU tests (tests/test_gpu_conversions.py).
  uint32_t words[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const uint32_t dw = (e < 8) ? v0[e / 2] : v1[(e - 8) / 2];
    const float xs[2] = {__uint_as_float(dw << 16), __uint_as_float(dw & 0xFFFF0000u)};
    float q[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      q[i] = __builtin_copysignf(element_quotient(xs[i], d, r, fast), xs[i]);
    switch ((e % 8) / 2) {
      case 0: words[e / 8] = pack_e2m1_pair<0>(words[e / 8], q[0], q[1]); break;
      case 1: words[e / 8] = pack_e2m1_pair<1>(words[e / 8], q[0], q[1]); break;
      case 2: words[e / 8] = pack_e2m1_pair<2>(words[e / 8], q[0], q[1]); break;
      default: words[e / 8] = pack_e2m1_pair<3>(words[e / 8], q[0], q[1]); break;
    }
  }
  u32x2_t outw = {words[0], words[1]};
  *reinterpret_cast<u32x2_t*>(packed8) = outw;
  *scale1 = (uint8_t)scode;
}

// grid: (encode workgroups, batch); threads stride over the 16-value blocks.
__global__ __launch_bounds__(kQThreads) void encode_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, const uint32_t* __restrict__ partial,
    int parts, uint8_t* __restrict__ packed, uint8_t* __restrict__ scales,
    float* __restrict__ gscale, uint32_t* __restrict__ d_status) {
  __shared__ uint32_t red[kQThreads / kWave];
  const int t = blockIdx.y;
  // fold this tensor's partial maxima (same order in every workgroup)
  uint32_t m = 0;
  for (int i = threadIdx.x; i < parts; i += kQThreads) {
    uint32_t v = partial[(int64_t)t * parts + i];
    m = m > v ? m : v;
  }
  m = block_max_u32(m, red);
  if (m >= 0x7F80u) {  // a NaN or infinity somewhere in this tensor
    if (blockIdx.x == 0 && threadIdx.x == 0 && d_status != nullptr)
      atomicOr(d_status, NVFP4_DSTATUS_NONFINITE);
    return;
  }
  const float amax = bf16_bits_to_float(m);
  const float g = amax / (kE2M1Max * kE4M3Max);
  if (blockIdx.x == 0 && threadIdx.x == 0) gscale[t] = g;

  const int64_t blocks16 = n * (k / 16);
  const int64_t elems = n * k;
  // kQUnroll blocks per thread and iteration, loaded before any is encoded,
  // so each wave keeps that many 32-byte loads in flight
  const int64_t stride = (int64_t)gridDim.x * kQThreads;
  for (int64_t b0 = (int64_t)blockIdx.x * kQThreads + threadIdx.x; b0 < blocks16;
       b0 += stride * kQUnroll) {
    u32x4_t v[kQUnroll][2];
#pragma unroll
    for (int i = 0; i < kQUnroll; ++i) {
      const int64_t b = b0 + i * stride;
      if (b < blocks16) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w + (int64_t)t * elems + b * 16);
        v[i][0] = __builtin_nontemporal_load(src);
        v[i][1] = __builtin_nontemporal_load(src + 1);
      }
    }
#pragma unroll
    for (int i = 0; i < kQUnroll; ++i) {
      const int64_t b = b0 + i * stride;
      if (b < blocks16) encode_block(v[i][0], v[i][1], g, packed + (int64_t)t * (elems / 2) + b * 8,
                                     scales + (int64_t)t * (elems / 16) + b);
    }
  }
}

int quantize_parts(int64_t n, int64_t k, int cu_count) {
  // enough workgroups per tensor to stream it at full bandwidth, but few
  // enough that folding the partials stays cheap
  const int64_t vecs = n * k / 8;
  int64_t parts = (vecs + kQThreads * 16 - 1) / (kQThreads * 16);
  int64_t cap = 4LL * cu_count;
  if (parts > cap) parts = cap;
  if (parts < 1) parts = 1;
  return (int)parts;
}

hipError_t launch_quantize(const uint16_t* w, int64_t batch, int64_t n, int64_t k,
                           uint8_t* packed, uint8_t* scales, float* gscale, uint32_t* d_status,
                           uint32_t* partial, int parts, hipStream_t stream) {
  dim3 g1(parts, (unsigned)batch);
  hipLaunchKernelGGL(amax_partial_kernel, g1, dim3(kQThreads), 0, stream, w, n * k, partial,
                     parts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // encode workgroups: enough to cover the CUs several times over, each
  // striding over many blocks so the partials are folded few times
  const int64_t blocks16 = n * (k / 16);
  const int64_t wgs =
      std::min<int64_t>((blocks16 + kQThreads * kQUnroll - 1) / (kQThreads * kQUnroll), 8 * 256);
  dim3 g2((unsigned)wgs, (unsigned)batch);
  hipLaunchKernelGGL(encode_kernel, g2, dim3(kQThreads), 0, stream, w, n, k, partial, parts,
                     packed, scales, gscale, d_status);
  return hipGetLastError();
}

}  // namespace nvfp4
