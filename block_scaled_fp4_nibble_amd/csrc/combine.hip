// combine.hip -- MoE combine: the scatter half of the routing-aware MoE layer
// ("The FP4 Frontier", Finding 5).  Each token's output is the router-weighted
// sum of the outputs of its top-k routed rows:
//   out[t][c] = sum_j w[t][j] * y[rows[t][j]][c]   (j in order, FP32, rounded once)
// A slot with rows[t][j] < 0 contributes nothing.  Deterministic: no atomics,
// the sum order is fixed.  HBM-bound: each routed row is read once and each
// token row written once.
#include "nvfp4_internal.hpp"
#include "device_common.hpp"

namespace nvfp4 {

constexpr int kCombineThreads = 256;
constexpr int kCombineCols = 8;  // columns per thread (16 bytes of BF16)

template <bool YF32>
struct Raw8 {
  uint4 q[YF32 ? 2 : 1];
};

template <bool YF32>
__device__ __forceinline__ Raw8<YF32> load8(const void* y, int64_t off) {
  Raw8<YF32> r;
  if constexpr (YF32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(y) + off);
    r.q[0] = p[0];
    r.q[1] = p[1];
  } else {
    r.q[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y) + off);
  }
  return r;
}

template <bool YF32>
__device__ __forceinline__ void widen8(const Raw8<YF32>& r, float (&v)[8]) {
  if constexpr (YF32) {
    const uint32_t u[8] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w,
                           r.q[1].x, r.q[1].y, r.q[1].z, r.q[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(u[i]);
  } else {
    const uint32_t u[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}

// One workgroup per (token, 2048-column chunk); thread i covers 8 columns.
// The slots are taken 8 at a time: their row ids and weights are uniform over
// the workgroup (scalar loads), the 8 row loads are all issued before the
// first is summed, and the sum runs in slot order.
template <bool YF32, bool OF32>
__global__ __launch_bounds__(kCombineThreads) void moe_combine_kernel(
    const void* y, int64_t rows, const int32_t* token_rows, const float* w, int topk, int n,
    int chunks, void* out, uint32_t* d_status) {
  const int64_t t = blockIdx.x / chunks;
  const int c = ((int)(blockIdx.x % chunks) * kCombineThreads + (int)threadIdx.x) * kCombineCols;
  const bool col_ok = c < n;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  for (int j0 = 0; j0 < topk; j0 += 8) {
    int r[8];
    float wt[8];
    bool ok[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q;
      r[q] = j < topk ? token_rows[t * topk + j] : -1;
      wt[q] = j < topk ? w[t * topk + j] : 0.f;
      bad |= r[q] >= rows;
      ok[q] = r[q] >= 0 && r[q] < rows;
    }
    bool any = false;
#pragma unroll
    for (int q = 0; q < 8; ++q) any |= ok[q];
    if (!any || !col_ok) continue;
    // unconditional loads (an empty slot reads row 0, which exists since one
    // slot is valid) so that no branch separates them; the empty slots are
    // then skipped in the sum
    Raw8<YF32> raw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) raw[q] = load8<YF32>(y, (int64_t)(ok[q] ? r[q] : 0) * n + c);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (ok[q]) {
        float v[8];
        widen8<YF32>(raw[q], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wt[q] * v[i];
      }
    }
  }
  if (bad && threadIdx.x == 0 && (blockIdx.x % chunks) == 0 && d_status != nullptr)
    atomicOr(d_status, NVFP4_DSTATUS_BAD_INDEX);
  if (!col_ok) return;
  const int64_t o = t * n + c;
  if (OF32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + o);
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      q[i] = float_to_bf16_rne(acc[2 * i]) | (float_to_bf16_rne(acc[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o) = make_uint4(q[0], q[1], q[2], q[3]);
  }
}

hipError_t launch_moe_combine(const void* y, bool y_f32, int64_t rows, const int32_t* token_rows,
                              const float* w, int64_t tokens, int topk, int n, void* out,
                              bool out_f32, uint32_t* d_status, hipStream_t stream) {
  const int chunks = (n + kCombineThreads * kCombineCols - 1) / (kCombineThreads * kCombineCols);
  const dim3 grid((unsigned)(tokens * chunks));
#define NVFP4_COMBINE(YF, OF)                                                               \
  hipLaunchKernelGGL((moe_combine_kernel<YF, OF>), grid, dim3(kCombineThreads), 0, stream, y, \
                     rows, token_rows, w, topk, n, chunks, out, d_status)
  if (y_f32) {
    if (out_f32) NVFP4_COMBINE(true, true);
    else NVFP4_COMBINE(true, false);
  } else {
    if (out_f32) NVFP4_COMBINE(false, true);
    else NVFP4_COMBINE(false, false);
  }
#undef NVFP4_COMBINE
  return hipGetLastError();
}

}  // namespace nvfp4
