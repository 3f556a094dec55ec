// api.hip -- the C ABI of libnvfp4.so: argument checks, schedule choice and
// launches.  Declarations and the contract are in include/nvfp4.h.
//
// Boundary lesson from the pages: a FP4 GEMM backend that launched, finished
// and silently returned all zeros on unsupported hardware ("The SM120 FP4
// GEMM Kernel Investigation", section "The Breaking Point: FlashInfer #2577")
// and tile configurations that failed to initialize ("The Tile That Didn't
// Fit", section "Why Tile Size Matters for FP4 Performance").  Here every
// call either enqueues the complete computation or returns a non-OK status
// without enqueuing anything.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "nvfp4_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices] = {0};
std::mutex g_mu;

// Compute-unit count of the current device (cached per device).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cu_count[dev] > 0) return g_cu_count[dev];
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      v <= 0)
    v = 256;
  std::lock_guard<std::mutex> lk(g_mu);
  g_cu_count[dev] = v;
  return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kInt31 = (int64_t)1 << 31;

nvfp4_status_t hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

nvfp4_status_t check_k(int64_t k) {
  if (k < 16 || (k % 16) != 0 || k >= kInt31) return NVFP4_ERR_INVALID_ARGUMENT;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(nvfp4_status_t s) {
  switch (s) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_INVALID_ARGUMENT: return "NVFP4_ERR_INVALID_ARGUMENT";
    case NVFP4_ERR_MISALIGNED: return "NVFP4_ERR_MISALIGNED";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP";
  }
  return "NVFP4_ERR_UNKNOWN";
}

int nvfp4_version(void) { return 100; }

size_t nvfp4_workspace_counter_bytes(void) { return nvfp4::kCounterBytes; }

nvfp4_status_t nvfp4_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (ws_bytes == 0) return NVFP4_OK;
  if (workspace == nullptr) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace)) return NVFP4_ERR_MISALIGNED;
  const size_t bytes = std::min(ws_bytes, nvfp4::kCounterBytes) / 16 * 16;
  return hip_status(
      nvfp4::launch_fill_zero(workspace, bytes, reinterpret_cast<hipStream_t>(stream)));
}

// ---- quantize --------------------------------------------------------------

size_t nvfp4_quantize_workspace_size(int64_t batch, int64_t n, int64_t k) {
  if (batch <= 0 || n <= 0 || check_k(k) != NVFP4_OK) return 0;
  const int parts = nvfp4::quantize_parts(n, k, cu_count());
  return (size_t)batch * parts * sizeof(uint32_t);
}

nvfp4_status_t nvfp4_quantize(const void* w_bf16, int64_t batch, int64_t n, int64_t k,
                              uint8_t* packed, uint8_t* scales, float* global_scale,
                              uint32_t* d_status, void* workspace, size_t ws_bytes,
                              void* stream) {
  if (batch < 0 || n < 1 || check_k(k) != NVFP4_OK) return NVFP4_ERR_INVALID_ARGUMENT;
  if (batch == 0) return NVFP4_OK;
  if (!w_bf16 || !packed || !scales || !global_scale) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned16(w_bf16) || !aligned16(packed) || !aligned16(scales) ||
      (reinterpret_cast<uintptr_t>(global_scale) & 3u) != 0)
    return NVFP4_ERR_MISALIGNED;
  if (batch > 65535) return NVFP4_ERR_UNSUPPORTED;
  if (n * (k / 16) / 256 >= kInt31) return NVFP4_ERR_UNSUPPORTED;
  const int parts = nvfp4::quantize_parts(n, k, cu_count());
  const size_t need = (size_t)batch * parts * sizeof(uint32_t);
  if (workspace == nullptr || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERR_MISALIGNED;
  return hip_status(nvfp4::launch_quantize(
      static_cast<const uint16_t*>(w_bf16), batch, n, k, packed, scales, global_scale, d_status,
      static_cast<uint32_t*>(workspace), parts, reinterpret_cast<hipStream_t>(stream)));
}

// ---- GEMM ------------------------------------------------------------------

static nvfp4_status_t check_gemm_common(const void* x, int64_t rows, int64_t n, int64_t k,
                                       const void* packed, const void* scales, const void* g,
                                       const void* y, nvfp4_out_t out) {
  if (rows < 0 || n < 1 || check_k(k) != NVFP4_OK) return NVFP4_ERR_INVALID_ARGUMENT;
  if (out != NVFP4_OUT_BF16 && out != NVFP4_OUT_F32) return NVFP4_ERR_INVALID_ARGUMENT;
  if (rows >= kInt31 || n >= kInt31) return NVFP4_ERR_UNSUPPORTED;
  // per-expert weight bytes are addressed with 32-bit buffer offsets
  if (n * (k / 2) >= kInt31 || k >= ((int64_t)1 << 24)) return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0) return NVFP4_OK;
  if (!x || !packed || !scales || !g || !y) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(g) & 3u) != 0)
    return NVFP4_ERR_MISALIGNED;
  return NVFP4_OK;
}

size_t nvfp4_gemm_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || check_k(k) != NVFP4_OK) return 0;
  return nvfp4::plan_gemm(m, 1, n, k, false, cu_count()).ws_bytes;
}

size_t nvfp4_grouped_gemm_workspace_size(int64_t rows, int64_t num_experts, int64_t n,
                                         int64_t k) {
  if (rows <= 0 || num_experts <= 0 || n <= 0 || check_k(k) != NVFP4_OK) return 0;
  return nvfp4::plan_gemm(rows, num_experts, n, k, true, cu_count()).ws_bytes;
}

const char* nvfp4_kernel_name(int64_t rows, int64_t num_experts, int64_t n, int64_t k,
                              int32_t grouped, int32_t gather) {
  if (rows <= 0 || num_experts <= 0 || n <= 0 || check_k(k) != NVFP4_OK) return "";
  const nvfp4::GemmPlan pl =
      nvfp4::plan_gemm(rows, num_experts, n, k, grouped != 0, cu_count());
  return nvfp4::plan_kernel_name(pl, grouped != 0 && gather != 0);
}

static nvfp4_status_t run_gemm(const void* x, int64_t rows, const int32_t* offsets, int64_t E,
                               int64_t n, int64_t k, const uint8_t* packed,
                               const uint8_t* scales, const float* g, void* y, nvfp4_out_t out,
                               uint32_t* d_status, void* workspace, size_t ws_bytes,
                               hipStream_t stream, bool grouped, int act = 0,
                               const int32_t* row_index = nullptr, int64_t x_rows = 0) {
  const nvfp4::GemmPlan pl = nvfp4::plan_gemm(rows, E, n, k, grouped, cu_count());
  // the SiLU(gate) * up epilogue pairs each wave's column tiles; a kernel
  // configuration with one tile per wave cannot serve it (never silent)
  if (act != 0 && !nvfp4::plan_pairs_tiles(pl)) return NVFP4_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0) {
    if (workspace == nullptr || ws_bytes < pl.ws_bytes) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_MISALIGNED;
  }
  nvfp4::GemmParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = packed;
  p.s = scales;
  p.g = g;
  p.offsets = offsets;
  p.y = y;
  p.counters = pl.splits > 1 ? static_cast<uint32_t*>(workspace) : nullptr;
  p.partials = pl.splits > 1
                   ? reinterpret_cast<float*>(static_cast<char*>(workspace) + nvfp4::kCounterBytes)
                   : nullptr;
  p.d_status = d_status;
  p.rows = rows;
  p.num_experts = (int32_t)E;
  p.n = (int32_t)n;
  p.k = (int32_t)k;
  p.splits = pl.splits;
  p.k_split = pl.k_split;
  p.n_tiles = pl.n_tiles;
  p.total_units = -1;
  p.out_f32 = out == NVFP4_OUT_F32 ? 1 : 0;
  p.act = act;
  p.row_index = row_index;
  p.x_rows = (int32_t)x_rows;
  return hip_status(nvfp4::launch_gemm(pl, p, stream));
}

nvfp4_status_t nvfp4_gemm(const void* x_bf16, int64_t m, int64_t n, int64_t k,
                          const uint8_t* packed, const uint8_t* scales,
                          const float* global_scale, void* y, nvfp4_out_t out, void* workspace,
                          size_t ws_bytes, void* stream) {
  nvfp4_status_t st = check_gemm_common(x_bf16, m, n, k, packed, scales, global_scale, y, out);
  if (st != NVFP4_OK || m == 0) return st;
  return run_gemm(x_bf16, m, nullptr, 1, n, k, packed, scales, global_scale, y, out, nullptr,
                  workspace, ws_bytes, reinterpret_cast<hipStream_t>(stream), false);
}

nvfp4_status_t nvfp4_grouped_gemm(const void* x_bf16, int64_t rows,
                                  const int32_t* expert_offsets, int64_t num_experts, int64_t n,
                                  int64_t k, const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scales, void* y, nvfp4_out_t out,
                                  uint32_t* d_status, void* workspace, size_t ws_bytes,
                                  void* stream) {
  if (num_experts < 1) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_experts > NVFP4_MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
  nvfp4_status_t st =
      check_gemm_common(x_bf16, rows, n, k, packed, scales, global_scales, y, out);
  if (st != NVFP4_OK || rows == 0) return st;
  if (expert_offsets == nullptr) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(expert_offsets) & 3u) != 0) return NVFP4_ERR_MISALIGNED;
  return run_gemm(x_bf16, rows, expert_offsets, num_experts, n, k, packed, scales,
                  global_scales, y, out, d_status, workspace, ws_bytes,
                  reinterpret_cast<hipStream_t>(stream), true);
}

nvfp4_status_t nvfp4_grouped_gemm_swiglu(const void* x_bf16, int64_t rows,
                                         const int32_t* expert_offsets, int64_t num_experts,
                                         int64_t n, int64_t k, const uint8_t* packed,
                                         const uint8_t* scales, const float* global_scales,
                                         void* h, nvfp4_out_t out, uint32_t* d_status,
                                         void* workspace, size_t ws_bytes, void* stream) {
  if (num_experts < 1) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_experts > NVFP4_MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
  if (n % 32 != 0) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status_t st =
      check_gemm_common(x_bf16, rows, n, k, packed, scales, global_scales, h, out);
  if (st != NVFP4_OK || rows == 0) return st;
  if (expert_offsets == nullptr) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(expert_offsets) & 3u) != 0) return NVFP4_ERR_MISALIGNED;
  return run_gemm(x_bf16, rows, expert_offsets, num_experts, n, k, packed, scales,
                  global_scales, h, out, d_status, workspace, ws_bytes,
                  reinterpret_cast<hipStream_t>(stream), true, 1);
}

// ---- MoE MLP in one launch -----------------------------------------------------

namespace {
int env_or(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

// The two products of a fused MoE MLP and the launch that runs both.
struct MlpPlan {
  nvfp4::GemmPlan up, down;
  bool ok;
  int grid;
  size_t ws_bytes;  // the GEMM counter region (left untouched, so the buffer can be
                    // shared with the GEMM calls), then per-row-tile counts of stored
                    // gate_up column tiles
};

MlpPlan plan_mlp(int64_t rows, int64_t E, int64_t d_model, int64_t d_ff) {
  MlpPlan m{};
  const int cus = cu_count();
  // no K split: the down tiles of the same launch keep the CUs busy
  m.up = nvfp4::plan_gemm(rows, E, 2 * d_ff, d_model, true, cus, false);
  m.down = nvfp4::plan_gemm(rows, E, d_model, d_ff, true, cus, false);
  m.ok = nvfp4::plan_fusable(m.up, m.down) && nvfp4::plan_pairs_tiles(m.up);
  if (!m.ok) return m;
  // every workgroup must be resident at once (a down tile waits for gate_up
  // tiles of other workgroups): at most one per resident slot of the fused
  // kernel itself
  const int slots = cus * nvfp4::fused_occupancy(m.up);
  m.grid = std::max(1, std::min(slots, std::max(m.up.grid, m.down.grid)));
  const int64_t row_tiles = (rows + m.up.bm - 1) / m.up.bm + std::min<int64_t>(E, rows);
  m.ws_bytes = nvfp4::kCounterBytes + (((size_t)row_tiles * 4 + 255) & ~(size_t)255);
  return m;
}

// 64-column multiples (whole 16-byte epilogue pieces, even 16-column tile
// pairs for SiLU(gate) * up); widths the LDS-staged epilogue covers (the
// first product's tiles are stored with device-scope stores only there)
bool mlp_shape_ok(int64_t d_model, int64_t d_ff) {
  return d_model % 64 == 0 && d_ff % 64 == 0 && 2 * d_ff <= nvfp4::kFixedStoreMaxN &&
         d_model <= nvfp4::kFixedStoreMaxN;
}
}  // namespace

size_t nvfp4_grouped_mlp_workspace_size(int64_t rows, int64_t num_experts, int64_t d_model,
                                        int64_t d_ff) {
  if (rows <= 0 || num_experts <= 0 || num_experts > NVFP4_MAX_EXPERTS || d_model <= 0 ||
      d_ff <= 0 || !mlp_shape_ok(d_model, d_ff))
    return 0;
  const MlpPlan m = plan_mlp(rows, num_experts, d_model, d_ff);
  return m.ok ? m.ws_bytes : 0;
}

nvfp4_status_t nvfp4_grouped_mlp(const void* x_bf16, int64_t rows,
                                 const int32_t* expert_offsets, int64_t num_experts,
                                 int64_t d_model, int64_t d_ff, const uint8_t* up_packed,
                                 const uint8_t* up_scales, const float* up_global,
                                 const uint8_t* down_packed, const uint8_t* down_scales,
                                 const float* down_global, void* h, void* y, nvfp4_out_t out,
                                 uint32_t* d_status, void* workspace, size_t ws_bytes,
                                 void* stream) {
  if (num_experts < 1 || d_model < 1 || d_ff < 1) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_experts > NVFP4_MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
  nvfp4_status_t st = check_gemm_common(x_bf16, rows, 2 * d_ff, d_model, up_packed, up_scales,
                                        up_global, h, NVFP4_OUT_BF16);
  if (st != NVFP4_OK) return st;
  st = check_gemm_common(h, rows, d_model, d_ff, down_packed, down_scales, down_global, y, out);
  if (st != NVFP4_OK) return st;
  if (!mlp_shape_ok(d_model, d_ff)) return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0) return NVFP4_OK;
  if (expert_offsets == nullptr) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(expert_offsets) & 3u) != 0) return NVFP4_ERR_MISALIGNED;
  const MlpPlan m = plan_mlp(rows, num_experts, d_model, d_ff);
  if (!m.ok) return NVFP4_ERR_UNSUPPORTED;
  if (workspace == nullptr || ws_bytes < m.ws_bytes) return NVFP4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERR_MISALIGNED;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  nvfp4::GemmParams p{};
  p.x = static_cast<const uint16_t*>(x_bf16);
  p.w = up_packed;
  p.s = up_scales;
  p.g = up_global;
  p.offsets = expert_offsets;
  p.y = h;
  p.d_status = d_status;
  p.rows = rows;
  p.num_experts = (int32_t)num_experts;
  p.n = (int32_t)(2 * d_ff);
  p.k = (int32_t)d_model;
  p.splits = 1;
  p.k_split = m.up.k_split;
  p.n_tiles = m.up.n_tiles;
  p.total_units = -1;
  p.out_f32 = 0;
  p.act = 1;
  p.w2 = down_packed;
  p.s2 = down_scales;
  p.g2 = down_global;
  p.y2 = y;
  p.n2 = (int32_t)d_model;
  p.k2 = (int32_t)d_ff;
  p.n_tiles2 = m.down.n_tiles;
  p.out2_f32 = out == NVFP4_OUT_F32 ? 1 : 0;
  uint32_t* counts =
      reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + nvfp4::kCounterBytes);
  p.rt_counters = counts;
  // a wait polls about every microsecond: 2^17 polls are ~0.1 s, far beyond
  // any wait of a resident grid.  NVFP4_MLP_SPIN and NVFP4_MLP_WAIT_EXTRA are
  // test hooks (a tiny limit, and a target no count reaches, force the
  // give-up path while every kernel still ends normally).
  p.spin_limit = std::max(0, env_or("NVFP4_MLP_SPIN", 1 << 17));
  p.wait_extra = std::max(0, env_or("NVFP4_MLP_WAIT_EXTRA", 0));
  if (nvfp4::launch_fill_zero(counts, m.ws_bytes - nvfp4::kCounterBytes, s) != hipSuccess)
    return NVFP4_ERR_HIP;
  return hip_status(nvfp4::launch_gemm_fused(m.up, m.grid, p, s));
}

const char* nvfp4_grouped_mlp_kernel_name(int64_t rows, int64_t num_experts, int64_t d_model,
                                          int64_t d_ff) {
  if (rows <= 0 || num_experts <= 0 || d_model <= 0 || d_ff <= 0 ||
      !mlp_shape_ok(d_model, d_ff))
    return "";
  const MlpPlan m = plan_mlp(rows, num_experts, d_model, d_ff);
  return m.ok ? nvfp4::fused_kernel_name(m.up) : "";
}

// ---- GEMM without allocation ------------------------------------------------

namespace {
// Scratch of nvfp4_gemm_noalloc: the split-K tile counters (the first
// kCounterBytes, zero at rest) and the partial tiles, in one array per device
// that the library's code object holds from load to process end.
constexpr size_t kScratchBytes = NVFP4_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > nvfp4::kCounterBytes, "counters fit the scratch");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Per device: the scratch array's device address (in host code the array's
// name is only a stand-in for the symbol) once looked up and its counter
// region zeroed.
void* g_scratch_ptr[kMaxDevices] = {nullptr};

nvfp4_status_t scratch_ptr(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return NVFP4_ERR_HIP;
    // counters must start at zero (a fill kernel, not a memset node, so this
    // may run under stream capture); completed calls leave them zero
    if (nvfp4::launch_fill_zero(ptr, nvfp4::kCounterBytes, stream) != hipSuccess)
      return NVFP4_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}
}  // namespace

nvfp4_status_t nvfp4_gemm_noalloc(const void* x_bf16, int64_t m, int64_t n, int64_t k,
                                  const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scale, void* y, nvfp4_out_t out,
                                  void* stream) {
  nvfp4_status_t st = check_gemm_common(x_bf16, m, n, k, packed, scales, global_scale, y, out);
  if (st != NVFP4_OK || m == 0) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t need = nvfp4::plan_gemm(m, 1, n, k, false, cu_count()).ws_bytes;
  if (need > kScratchBytes) return NVFP4_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_ptr(s, &ws);
    if (st != NVFP4_OK) return st;
  }
  return run_gemm(x_bf16, m, nullptr, 1, n, k, packed, scales, global_scale, y, out, nullptr, ws,
                  need > 0 ? kScratchBytes : 0, s, false);
}

// ---- W4A4 -----------------------------------------------------------------

namespace {
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
// Workspace of a W4A4 call: the GEMM's own workspace first (split-K counters
// must sit at its start), then the decoded BF16 activations, then the
// per-expert products of the global scales.  The counter region is reserved
// even when this call does not split K: a workspace serves calls of every
// shape, and the counters must stay zero between them.
struct W4A4Layout {
  size_t gemm, x_off, g_off, total;
};
W4A4Layout w4a4_layout(int64_t rows, int64_t E, int64_t n, int64_t k, bool grouped) {
  W4A4Layout l;
  l.gemm = nvfp4::plan_gemm(rows, E, n, k, grouped, cu_count()).ws_bytes;
  l.x_off = align256(std::max(l.gemm, nvfp4::kCounterBytes));
  l.g_off = l.x_off + align256((size_t)rows * (size_t)k * 2);
  l.total = l.g_off + align256((size_t)E * 4);
  return l;
}
}  // namespace

size_t nvfp4_gemm_w4a4_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || check_k(k) != NVFP4_OK) return 0;
  return w4a4_layout(m, 1, n, k, false).total;
}

size_t nvfp4_grouped_gemm_w4a4_workspace_size(int64_t rows, int64_t num_experts, int64_t n,
                                              int64_t k) {
  if (rows <= 0 || num_experts <= 0 || n <= 0 || check_k(k) != NVFP4_OK) return 0;
  return w4a4_layout(rows, num_experts, n, k, true).total;
}

static nvfp4_status_t run_w4a4(const uint8_t* x_packed, const uint8_t* x_scales, const float* x_g,
                               int64_t rows, const int32_t* offsets, int64_t E, int64_t n,
                               int64_t k, const uint8_t* packed, const uint8_t* scales,
                               const float* g, void* y, nvfp4_out_t out, uint32_t* d_status,
                               void* workspace, size_t ws_bytes, hipStream_t stream,
                               bool grouped) {
  if (!x_scales || !x_g) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(x_g) & 3u) != 0) return NVFP4_ERR_MISALIGNED;
  const W4A4Layout l = w4a4_layout(rows, E, n, k, grouped);
  if (workspace == nullptr || ws_bytes < l.total) return NVFP4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERR_MISALIGNED;
  char* ws = static_cast<char*>(workspace);
  uint16_t* x_bf16 = reinterpret_cast<uint16_t*>(ws + l.x_off);
  float* g_comb = reinterpret_cast<float*>(ws + l.g_off);
  hipError_t err = nvfp4::launch_dequant_rows(x_packed, x_scales, rows, k, x_bf16, x_g, g,
                                              g_comb, (int)E, stream);
  if (err != hipSuccess) return hip_status(err);
  return run_gemm(x_bf16, rows, offsets, E, n, k, packed, scales, g_comb, y, out, d_status, ws,
                  l.gemm, stream, grouped);
}

nvfp4_status_t nvfp4_gemm_w4a4(const uint8_t* x_packed, const uint8_t* x_scales,
                               const float* x_global_scale, int64_t m, int64_t n, int64_t k,
                               const uint8_t* packed, const uint8_t* scales,
                               const float* global_scale, void* y, nvfp4_out_t out,
                               void* workspace, size_t ws_bytes, void* stream) {
  nvfp4_status_t st = check_gemm_common(x_packed, m, n, k, packed, scales, global_scale, y, out);
  if (st != NVFP4_OK || m == 0) return st;
  return run_w4a4(x_packed, x_scales, x_global_scale, m, nullptr, 1, n, k, packed, scales,
                  global_scale, y, out, nullptr, workspace, ws_bytes,
                  reinterpret_cast<hipStream_t>(stream), false);
}

nvfp4_status_t nvfp4_grouped_gemm_w4a4(const uint8_t* x_packed, const uint8_t* x_scales,
                                       const float* x_global_scale, int64_t rows,
                                       const int32_t* expert_offsets, int64_t num_experts,
                                       int64_t n, int64_t k, const uint8_t* packed,
                                       const uint8_t* scales, const float* global_scales,
                                       void* y, nvfp4_out_t out, uint32_t* d_status,
                                       void* workspace, size_t ws_bytes, void* stream) {
  if (num_experts < 1) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_experts > NVFP4_MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
  nvfp4_status_t st =
      check_gemm_common(x_packed, rows, n, k, packed, scales, global_scales, y, out);
  if (st != NVFP4_OK || rows == 0) return st;
  if (!expert_offsets) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(expert_offsets) & 3u) != 0) return NVFP4_ERR_MISALIGNED;
  return run_w4a4(x_packed, x_scales, x_global_scale, rows, expert_offsets, num_experts, n, k,
                  packed, scales, global_scales, y, out, d_status, workspace, ws_bytes,
                  reinterpret_cast<hipStream_t>(stream), true);
}

nvfp4_status_t nvfp4_moe_combine(const void* y, nvfp4_out_t y_type, int64_t rows,
                                 const int32_t* token_rows, const float* weights,
                                 int64_t tokens, int64_t topk, int64_t n, void* out,
                                 nvfp4_out_t out_type, uint32_t* d_status, void* stream) {
  if (tokens < 0 || rows < 0 || n < 1 || n % 8 != 0 || topk < 1 || topk > 64)
    return NVFP4_ERR_INVALID_ARGUMENT;
  if ((y_type != NVFP4_OUT_BF16 && y_type != NVFP4_OUT_F32) ||
      (out_type != NVFP4_OUT_BF16 && out_type != NVFP4_OUT_F32))
    return NVFP4_ERR_INVALID_ARGUMENT;
  if (n >= kInt31 || rows >= kInt31 || tokens >= kInt31 / 64 ||
      tokens * ((n + 2047) / 2048) >= kInt31)  // one workgroup per 2048-column chunk
    return NVFP4_ERR_UNSUPPORTED;
  if (tokens == 0) return NVFP4_OK;
  if (!y || !token_rows || !weights || !out) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned16(y) || !aligned16(out) || (reinterpret_cast<uintptr_t>(token_rows) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(weights) & 3u) != 0)
    return NVFP4_ERR_MISALIGNED;
  return hip_status(nvfp4::launch_moe_combine(
      y, y_type == NVFP4_OUT_F32, rows, token_rows, weights, tokens, (int)topk, (int)n, out,
      out_type == NVFP4_OUT_F32, d_status, reinterpret_cast<hipStream_t>(stream)));
}

nvfp4_status_t nvfp4_grouped_gemm_gather(const void* x_bf16, int64_t x_rows,
                                         const int32_t* row_index, int64_t rows,
                                         const int32_t* expert_offsets, int64_t num_experts,
                                         int64_t n, int64_t k, const uint8_t* packed,
                                         const uint8_t* scales, const float* global_scales,
                                         void* y, nvfp4_out_t out, int32_t act,
                                         uint32_t* d_status, void* workspace, size_t ws_bytes,
                                         void* stream) {
  if (num_experts < 1 || x_rows < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_experts > NVFP4_MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
  if (act != 0 && act != 1) return NVFP4_ERR_INVALID_ARGUMENT;
  if (act == 1 && n % 32 != 0) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status_t st =
      check_gemm_common(x_bf16, rows, n, k, packed, scales, global_scales, y, out);
  if (st != NVFP4_OK || rows == 0) return st;
  if (expert_offsets == nullptr || row_index == nullptr || x_rows == 0)
    return NVFP4_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(expert_offsets) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(row_index) & 3u) != 0)
    return NVFP4_ERR_MISALIGNED;
  // buffer offsets into x are 32-bit
  if (x_rows > INT32_MAX || (uint64_t)x_rows * (uint64_t)k * 2u > 0xffffffffull)
    return NVFP4_ERR_UNSUPPORTED;
  return run_gemm(x_bf16, rows, expert_offsets, num_experts, n, k, packed, scales,
                  global_scales, y, out, d_status, workspace, ws_bytes,
                  reinterpret_cast<hipStream_t>(stream), true, act, row_index, x_rows);
}

}  // extern "C"
