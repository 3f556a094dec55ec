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
//   (deterministic, no atomics), derives g, then each thread encodes one
//   16-value block: 32 bytes in, 8 packed bytes + 1 scale byte out.
// Both passes stream W with 16-byte loads; W is read twice from HBM.
#include "device_common.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

constexpr int kQThreads = 256;

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
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < vecs;
       i += (int64_t)parts * kQThreads) {
    m = max_mag_bits(__builtin_nontemporal_load(src + i), m);
  }
  uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  m = lo > hi ? lo : hi;
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[(int64_t)t * parts + blockIdx.x] = m;
}

// grid: (ceil(blocks16 / kQThreads), batch); one thread per 16-value block.
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
  const int64_t b = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (b >= blocks16) return;
  const int64_t elems = n * k;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w + (int64_t)t * elems + b * 16);
  u32x4_t v0 = __builtin_nontemporal_load(src);
  u32x4_t v1 = __builtin_nontemporal_load(src + 1);
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

  uint32_t words[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t dw = (e < 8) ? v0[e / 2] : v1[(e - 8) / 2];
    const uint32_t h = (e & 1) ? (dw >> 16) : (dw & 0xFFFFu);
    const float x = bf16_bits_to_float(h & 0x7FFFu);
    uint32_t mag = 0;
    if (d != 0.0f) mag = encode_e2m1_mag(x / d);
    const uint32_t code = ((h >> 15) << 3) | mag;
    words[e / 8] |= code << (4 * (e % 8));
  }
  u32x2_t outw = {words[0], words[1]};
  *reinterpret_cast<u32x2_t*>(packed + (int64_t)t * (elems / 2) + b * 8) = outw;
  scales[(int64_t)t * (elems / 16) + b] = (uint8_t)scode;
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
  const int64_t blocks16 = n * (k / 16);
  dim3 g2((unsigned)((blocks16 + kQThreads - 1) / kQThreads), (unsigned)batch);
  hipLaunchKernelGGL(encode_kernel, g2, dim3(kQThreads), 0, stream, w, n, k, partial, parts,
                     packed, scales, gscale, d_status);
  return hipGetLastError();
}

}  // namespace nvfp4
