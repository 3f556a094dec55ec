// w4a4.hip -- activations in NVFP4 too (W4A4).
//
// The pages' FP4 GEMMs keep block-scaled FP4 data and scale tiles for both
// operands ("The SM120 FP4 GEMM Kernel Investigation", section "The
// Comprehensive Synthesis: Message 6").  gfx950's scaled MFMA takes E8M0
// scales per 32 values, not E4M3 per 16, so the product stays on BF16 MFMA:
// the activations are decoded once per launch into BF16 (e2m1 x E4M3 is exact
// in BF16, the activation's global scale left out), and the W4A16 kernels run
// on them with the global scale g_w[e] * g_x.  This kernel does the decoding
// and forms those per-expert scale products.
#include <algorithm>

#include "device_common.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

constexpr int kDqThreads = 256;

// x_bf16[8 i .. 8 i + 7] = e2m1(packed dword i) * E4M3(scales[i / 2]): the
// flat element index 8 i lies in 16-block i / 2 of the same row since k is a
// multiple of 16.  Block 0 also writes g_out[e] = g_w[e] * g_x[0].
__global__ __launch_bounds__(kDqThreads) void dequant_rows_kernel(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales, int64_t groups,
    bf16x8_t* __restrict__ x_bf16, const float* __restrict__ g_x, const float* __restrict__ g_w,
    float* __restrict__ g_out, int num_experts) {
  const int64_t stride = (int64_t)gridDim.x * kDqThreads;
  for (int64_t i = (int64_t)blockIdx.x * kDqThreads + threadIdx.x; i < groups; i += stride)
    x_bf16[i] = dequant8(packed[i], decode_e4m3<0>(scales[i >> 1]));
  if (blockIdx.x == 0)
    for (int e = threadIdx.x; e < num_experts; e += kDqThreads) g_out[e] = g_w[e] * g_x[0];
}

hipError_t launch_dequant_rows(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                               int64_t k, uint16_t* x_bf16, const float* g_x, const float* g_w,
                               float* g_out, int num_experts, hipStream_t stream) {
  const int64_t groups = rows * k / 8;
  const int64_t wgs = std::max<int64_t>(
      1, std::min<int64_t>((groups + kDqThreads - 1) / kDqThreads, 8 * 256));
  hipLaunchKernelGGL(dequant_rows_kernel, dim3((unsigned)wgs), dim3(kDqThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(packed), scales, groups,
                     reinterpret_cast<bf16x8_t*>(x_bf16), g_x, g_w, g_out, num_experts);
  return hipGetLastError();
}

}  // namespace nvfp4
