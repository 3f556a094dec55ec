// conv_probe.hip -- test-only kernels that run the product's device
// conversion helpers (block_scaled_fp4_nibble_amd/csrc/device_common.hpp)
// over exhaustive input sets, so that the GPU tests can compare what the
// hardware conversions produce with the oracle's definitions.  Built into
// tests/gpu_probe/libnvfp4_probe.so; the product library does not contain or
// load any of it.
//
// The formats are those of the page "The Blackwell Architectural Split:
// NVFP4, Attention, and Consumer Silicon", section "Preserving precision --
// dual-tier scale handling": E2M1 elements, E4M3 block scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../block_scaled_fp4_nibble_amd/csrc/device_common.hpp"

using namespace nvfp4;

namespace {

// out[i] = code(x) | code(-x) << 4 for x = the FP32 pattern base + i, through
// the encoder's pack conversion (pack_e2m1_pair).
__global__ void e2m1_pack_kernel(uint32_t base, uint32_t n, uint8_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float x = __uint_as_float(base + i);
  out[i] = (uint8_t)(pack_e2m1_pair<0>(0u, x, -x) & 0xFFu);
}

// out[i] = encode_e4m3(x) for x = the FP32 pattern base + i (the block-scale
// encoder; it only ever sees finite non-negative values).
__global__ void e4m3_encode_kernel(uint32_t base, uint32_t n, uint8_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = (uint8_t)encode_e4m3(__uint_as_float(base + i));
}

// out[4 c + s] = decode_e4m3<s> of code c placed in byte s of a dword.
__global__ void e4m3_decode_kernel(float* __restrict__ out) {
  const uint32_t c = threadIdx.x;  // 256 threads
  out[4 * c + 0] = decode_e4m3<0>(c);
  out[4 * c + 1] = decode_e4m3<1>(c << 8);
  out[4 * c + 2] = decode_e4m3<2>(c << 16);
  out[4 * c + 3] = decode_e4m3<3>(c << 24);
}

// q[i] = element_quotient(x[i], d[i]) with the encoder's reciprocal choice.
__global__ void quotient_kernel(const float* __restrict__ x, const float* __restrict__ d,
                                float* __restrict__ q, uint32_t n) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float r;
  const bool fast = element_divisor(d[i], r);
  q[i] = element_quotient(x[i], d[i], r, fast);
}

// out[((s * nw) + j) * 8 + t] = float value of BF16 t of dequant8(w[j],
// decode(scale code s)), for the 127 finite non-negative scale codes s.
__global__ void dequant_kernel(const uint32_t* __restrict__ w, uint32_t nw,
                               float* __restrict__ out) {
  const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t s = blockIdx.y;
  if (j >= nw) return;
  const bf16x8_t v = dequant8(w[j], decode_e4m3<0>(s));
  u32x4_t bits;
  __builtin_memcpy(&bits, &v, sizeof(bits));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    out[((size_t)s * nw + j) * 8 + 2 * t] = __uint_as_float(bits[t] << 16);
    out[((size_t)s * nw + j) * 8 + 2 * t + 1] = __uint_as_float(bits[t] & 0xFFFF0000u);
  }
}

int err(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace

extern "C" {

int probe_e2m1_pack(uint32_t base, uint32_t n, uint8_t* out, void* stream) {
  hipLaunchKernelGGL(e2m1_pack_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), base, n, out);
  return err(hipGetLastError());
}

int probe_e4m3_encode(uint32_t base, uint32_t n, uint8_t* out, void* stream) {
  hipLaunchKernelGGL(e4m3_encode_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), base, n, out);
  return err(hipGetLastError());
}

int probe_e4m3_decode(float* out /* [1024] */, void* stream) {
  hipLaunchKernelGGL(e4m3_decode_kernel, dim3(1), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), out);
  return err(hipGetLastError());
}

int probe_quotient(const float* x, const float* d, float* q, uint32_t n, void* stream) {
  hipLaunchKernelGGL(quotient_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), x, d, q, n);
  return err(hipGetLastError());
}

int probe_dequant(const uint32_t* w, uint32_t nw, float* out /* [127][nw][8] */, void* stream) {
  hipLaunchKernelGGL(dequant_kernel, dim3((nw + 255) / 256, 127), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), w, nw, out);
  return err(hipGetLastError());
}

}  // extern "C"
