// nvfp4_internal.hpp -- launch interfaces shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

constexpr int kMaxExperts = NVFP4_MAX_EXPERTS;
// Split-K tile counters live in the first kCounterBytes of a GEMM workspace.
constexpr size_t kCounterBytes = 65536;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(uint32_t));
// Widest output for which a row tile's bytes (at most 64 rows of FP32) stay
// inside one 32-bit buffer range: the K-phase kernel's LDS-staged epilogue
// (and so the fused launch's device-scope stores) needs it.
constexpr int kFixedStoreMaxN = (1 << 23);

// ---- quantize -----------------------------------------------------------
int quantize_parts(int64_t n, int64_t k, int cu_count);
hipError_t launch_quantize(const uint16_t* w, int64_t batch, int64_t n, int64_t k,
                           uint8_t* packed, uint8_t* scales, float* gscale, uint32_t* d_status,
                           uint32_t* partial, int parts, hipStream_t stream);

// ---- GEMM ---------------------------------------------------------------
struct GemmParams {
  const uint16_t* x;        // [rows][k] bf16
  const uint8_t* w;         // [E][n][k/2]
  const uint8_t* s;         // [E][n][k/16]
  const float* g;           // [E]
  const int32_t* offsets;   // [E+1] on the device; nullptr: one segment of `rows`
  void* y;                  // [rows][n]
  float* partials;          // split-K partial tiles (nullptr when splits == 1)
  uint32_t* counters;       // split-K arrival counters (nullptr when splits == 1)
  uint32_t* d_status;       // may be nullptr
  int64_t rows;
  int32_t num_experts;
  int32_t n;
  int32_t k;
  int32_t splits;           // K splits per output tile
  int32_t k_split;          // K per split (multiple of 64 on the fast path, of 16 otherwise)
  int32_t n_tiles;          // ceil(n / column tile width of the chosen kernel)
  int32_t total_units;      // exact for dense, -1 for grouped (computed on device)
  int32_t out_f32;
  int32_t act;              // 1: y [rows][n / 2] = SiLU(gate) * up over 32-row gate/up groups
  const int32_t* row_index; // [rows]: routed row r reads x row row_index[r]; nullptr: row r
  int32_t x_rows;           // rows of x when row_index is given
  // The second product of a fused gate_up -> down launch (kernels built with
  // FUSED only): it reads the first product's output y as its activations.
  const uint8_t* w2;        // [E][n2][k2/2]
  const uint8_t* s2;        // [E][n2][k2/16]
  const float* g2;          // [E]
  void* y2;                 // [rows][n2]
  int32_t n2, k2, n_tiles2, out2_f32;
  uint32_t* rt_counters;    // per row tile of the first product: column tiles stored (zeroed)
  int32_t spin_limit;       // polls before a wait gives up
  int32_t wait_extra;       // added to every wait's target (0; a test sets 1 to force give-ups)
};

struct GemmPlan {
  int bm;        // rows per tile: 16, 32 or 64
  int kind;      // kernel configuration (see plan_gemm)
  int bn;        // columns per tile: 128 or 256
  int nslot;     // LDS ring slots of the K-phase kernel
  int dyn_lds;   // dynamic LDS bytes of the launch (the per-expert unit prefix)
  int splits;
  int k_split;
  int n_tiles;
  int max_tiles; // upper bound on output tiles (for counters / partials)
  int grid;
  bool fast;     // k % 64 == 0
  size_t ws_bytes;
};

// Dense products of at most kGemvMaxRows rows with k % 32 == 0 run on the
// dot-product kernel (gemv.hip), which stages the rows in LDS (at most
// kGemvMaxXBytes: six rows of K = 8192).
constexpr int kGemvMaxRows = 6;
// Both decode kernels run 8-wave workgroups.
constexpr int kGemvThreads = 512;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int64_t kGemvMaxXBytes = 98304;
// Dense products of 7 to 64 rows with k % 128 == 0 run on the split-K decode
// kernel (gemv.hip): units of kDskCols output columns by at most
// kDskMaxGroups 128-deep K groups.
constexpr int kDskCols = 64;
constexpr int kDskMaxGroups = 16;

// allow_split false: never split K (the fused gate_up -> down launch).
GemmPlan plan_gemm(int64_t rows, int64_t num_experts, int64_t n, int64_t k, bool grouped,
                   int cu_count, bool allow_split = true);
hipError_t launch_gemm(const GemmPlan& plan, const GemmParams& p, hipStream_t stream);
// Fused gate_up -> down launch: both products planned with the same K-phase
// kernel and no K split (false otherwise); `plan` is the first product's.
bool plan_fusable(const GemmPlan& up, const GemmPlan& down);
int fused_occupancy(const GemmPlan& plan);
const char* fused_kernel_name(const GemmPlan& plan);
hipError_t launch_gemm_fused(const GemmPlan& plan, int grid, const GemmParams& p,
                             hipStream_t stream);
const char* plan_kernel_name(const GemmPlan& plan, bool gather);
hipError_t launch_gemv(const GemmPlan& plan, const GemmParams& p, hipStream_t stream);
// True when every wave of the planned kernel ends with an even number of
// 16-column tiles (what the SiLU(gate) * up epilogue needs).
bool plan_pairs_tiles(const GemmPlan& plan);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);

// ---- W4A4: decode NVFP4 activations to BF16, form g_w[e] * g_x ----------------
hipError_t launch_dequant_rows(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                               int64_t k, uint16_t* x_bf16, const float* g_x, const float* g_w,
                               float* g_out, int num_experts, hipStream_t stream);

// ---- MoE combine -----------------------------------------------------------
hipError_t launch_moe_combine(const void* y, bool y_f32, int64_t rows, const int32_t* token_rows,
                              const float* w, int64_t tokens, int topk, int n, void* out,
                              bool out_f32, uint32_t* d_status, hipStream_t stream);

}  // namespace nvfp4
