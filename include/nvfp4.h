/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 weight-only GEMM library
 * (libnvfp4.so).
 *
 * What the library computes
 * -------------------------
 * NVFP4 weights: each value is an E2M1 4-bit float (1 sign, 2 exponent, 1
 * mantissa bit), and the format scales them in two tiers, one global FP32
 * scale per tensor and one FP8-E4M3 scale per block of 16 consecutive values
 * along K ("The Blackwell Architectural Split: NVFP4, Attention, and Consumer
 * Silicon", section "Preserving precision -- dual-tier scale handling"; the
 * A4Q section of the same page dequantizes exactly such 16-value blocks).
 * Activations and outputs are BF16 ("The SM120 FP4 GEMM Kernel
 * Investigation", section "The Context": 4-bit weights with BF16
 * activations).  The grouped GEMM runs every expert of a MoE layer in one
 * launch over per-expert token segments ("The FP4 Frontier", Finding 5:
 * grouped GEMM over all experts in a persistent kernel).
 *
 * Encoding (nvfp4_quantize), for one tensor W [n][k] in BF16:
 *   g      = fl32(amax(|W|) / 2688)                 (2688 = 6 * 448)
 *   s[b]   = E4M3_rne_sat(fl32(fl32(amax_b / 6) / g)), or 0 when g == 0
 *   d      = fl32(decode(s[b]) * g)
 *   code   = sign(w) << 3 | E2M1_rne_sat(fl32(|w| / d))   (magnitude 0 if d == 0)
 * "rne_sat": round to nearest, ties to the even code, clamp to the largest
 * finite value (448, resp. 6).  The sign bit is kept for values that round to
 * zero, so -0 encodes as 0x8.
 *
 * Product (nvfp4_gemm, nvfp4_grouped_gemm, nvfp4_grouped_gemm_swiglu,
 * nvfp4_grouped_gemm_gather):
 *   y[m][n] = g * sum_k x[m][k] * e2m1(code[n][k]) * decode(s[n][k/16])
 * Each e2m1 * E4M3 product is exact in BF16, so the kernels run BF16 MFMA with
 * FP32 accumulation and apply g once in the epilogue; the BF16 output is the
 * round-to-nearest-even of fl32(g * acc).
 *
 * Memory layout (all row-major, contiguous, device memory)
 * ---------------------------------------------------------
 *   W       bf16   [batch][n][k]
 *   packed  uint8  [batch][n][k/2]   byte j of a row: element 2j in the low
 *                                     nibble, element 2j+1 in the high nibble
 *   scales  uint8  [batch][n][k/16]  E4M3 (OCP "FN": max 448, no infinities)
 *   g       float  [batch]
 *   x       bf16   [m][k]            grouped: [rows][k], sorted by expert
 *   y       bf16 or float [m][n]     grouped: [rows][n]
 * Storage is exactly 4.5 bits per weight plus 32 bits per tensor ("The FP4
 * Frontier", Finding 6).
 *
 * Conventions
 * -----------
 *  - Ownership: the caller owns every buffer.  The library allocates no
 *    device or host memory; the state it keeps is cached device properties
 *    (compute-unit count) per device and, for nvfp4_gemm_noalloc only, one
 *    fixed scratch array per device that its code object holds.
 *  - Pointers are device pointers unless stated otherwise; `stream` is a
 *    hipStream_t (NULL means the default stream).  Every call only enqueues
 *    work on `stream` and returns without waiting for it.
 *  - Alignment: x, y, W, packed, scales and workspace must be 16-byte aligned,
 *    else NVFP4_ERR_MISALIGNED.  k must be a positive multiple of 16.  Any
 *    n >= 1, m >= 0 and k % 16 == 0 is supported; k % 64 == 0 takes the fast
 *    path.  m == 0 (or rows == 0) is a no-op that returns NVFP4_OK.
 *  - Errors the host can check are returned synchronously and nothing is
 *    enqueued.  A launch failure is returned as NVFP4_ERR_HIP.  No call ever
 *    "succeeds" without writing its outputs: an unsupported combination
 *    returns NVFP4_ERR_UNSUPPORTED.
 *  - Data-dependent errors set bits in the caller-provided device word
 *    `d_status` (may be NULL): NVFP4_DSTATUS_NONFINITE (quantize saw a NaN
 *    or infinity; outputs for that tensor are unspecified) and
 *    NVFP4_DSTATUS_BAD_OFFSETS (grouped GEMM saw offsets that are not a
 *    non-decreasing prefix array from 0 to rows; nothing is written to y)
 *    and NVFP4_DSTATUS_BAD_INDEX (a gathered row's index lies outside
 *    [0, x_rows); that row computes as if its activations were zero) and
 *    NVFP4_DSTATUS_WAIT_TIMEOUT (nvfp4_grouped_mlp: a workgroup's bounded
 *    wait for another workgroup's results gave up -- possible only when the
 *    launch's workgroups cannot all be resident at once; y is then
 *    unspecified).
 *    Bits are only ever set (atomic OR), never cleared, by the library.
 *  - Workspace: a device buffer of at least the size the matching
 *    *_workspace_size() function returns (0: pass NULL).  For the two GEMM
 *    calls, the first nvfp4_workspace_counter_bytes() bytes of a non-empty
 *    workspace hold split-K tile counters that must be zero before the first
 *    call that uses the buffer (nvfp4_workspace_init zeroes them); every
 *    completed call leaves them zero again.  The quantize workspace has no
 *    counters and needs no initialization.  Calls that may run concurrently
 *    need separate workspaces.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARGUMENT = 1, /* bad size, null pointer, k % 16 != 0 */
  NVFP4_ERR_MISALIGNED = 2,       /* a buffer is not 16-byte aligned */
  NVFP4_ERR_UNSUPPORTED = 3,      /* valid but not implemented (e.g. > 1024 experts) */
  NVFP4_ERR_WORKSPACE = 4,        /* workspace missing or too small */
  NVFP4_ERR_HIP = 5               /* the HIP runtime reported an error */
} nvfp4_status_t;

typedef enum { NVFP4_OUT_BF16 = 0, NVFP4_OUT_F32 = 1 } nvfp4_out_t;

#define NVFP4_DSTATUS_NONFINITE 1u
#define NVFP4_DSTATUS_BAD_OFFSETS 2u
#define NVFP4_DSTATUS_BAD_INDEX 4u
#define NVFP4_DSTATUS_WAIT_TIMEOUT 8u

/* Largest number of experts nvfp4_grouped_gemm accepts. */
#define NVFP4_MAX_EXPERTS 1024

/* Encode `batch` BF16 tensors W [batch][n][k] (two passes over W: tensor
 * amax, then block scales, element codes and nibble packing).  Writes
 * packed [batch][n][k/2], scales [batch][n][k/16] and global_scale [batch]
 * (device).  The encoding is bit-exact with the definition above: IEEE
 * binary32 division, no flush of subnormals.  Non-finite input sets
 * NVFP4_DSTATUS_NONFINITE in *d_status. */
nvfp4_status_t nvfp4_quantize(const void* w_bf16, int64_t batch, int64_t n, int64_t k,
                              uint8_t* packed, uint8_t* scales, float* global_scale,
                              uint32_t* d_status, void* workspace, size_t ws_bytes,
                              void* stream);

/* Dense W4A16 GEMM: y [m][n] = x [m][k] (bf16) times the decoded weight
 * (packed, scales, *global_scale -- a device pointer to one float).  The
 * schedule (rows per tile, split of K over workgroups for m <= 64) is chosen
 * from the shape and the device's compute-unit count; split-K partial sums
 * are reduced in a fixed order, so results are bitwise reproducible. */
nvfp4_status_t nvfp4_gemm(const void* x_bf16, int64_t m, int64_t n, int64_t k,
                          const uint8_t* packed, const uint8_t* scales,
                          const float* global_scale, void* y, nvfp4_out_t out,
                          void* workspace, size_t ws_bytes, void* stream);

/* Grouped (MoE) W4A16 GEMM.  x [rows][k] holds the routed token rows sorted
 * by expert; expert_offsets (device, int32 [num_experts + 1]) is the prefix
 * array: rows [offsets[e], offsets[e+1]) use expert e's weight
 * packed[e] [n][k/2], scales[e] [n][k/16], global_scales[e].  Empty experts
 * cost nothing and write nothing.  The offsets are read on the device (no
 * host synchronization); a persistent grid walks all (expert, row tile,
 * column tile, K split) work units.  Bad offsets set
 * NVFP4_DSTATUS_BAD_OFFSETS in *d_status (may be NULL) and write nothing. */
nvfp4_status_t nvfp4_grouped_gemm(const void* x_bf16, int64_t rows,
                                  const int32_t* expert_offsets, int64_t num_experts,
                                  int64_t n, int64_t k, const uint8_t* packed,
                                  const uint8_t* scales, const float* global_scales,
                                  void* y, nvfp4_out_t out, uint32_t* d_status,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Grouped gate_up GEMM with the SiLU(gate) * up epilogue of a MoE MLP ("The
 * FP4 Frontier", Finding 5: the fused gate_up GEMM + SiLU of the MoE layer).
 * Arguments and behaviour are those of nvfp4_grouped_gemm, except:
 *  - n (even, a multiple of 32) counts the fused weight's rows: each
 *    expert's packed[e] [n][k/2] and scales[e] [n][k/16] hold them in 32-row
 *    groups, 16 gate rows followed by the 16 up rows of the same outputs
 *    (output column c pairs rows 32 (c / 16) + c % 16 and that + 16);
 *    quantize the fused weight in that row order (one global scale per
 *    expert covers both halves);
 *  - the output h [rows][n / 2] (caller-allocated, 16-byte aligned) is
 *    h[r][c] = SiLU(g y_gate) * (g y_up) with SiLU(v) = v / (1 + e^-v),
 *    evaluated in FP32 on the FP32 accumulators and rounded once (RNE) for
 *    NVFP4_OUT_BF16;
 *  - n % 32 != 0 returns NVFP4_ERR_INVALID_ARGUMENT.
 * Workspace: nvfp4_grouped_gemm_workspace_size(rows, num_experts, n, k). */
nvfp4_status_t nvfp4_grouped_gemm_swiglu(const void* x_bf16, int64_t rows,
                                         const int32_t* expert_offsets, int64_t num_experts,
                                         int64_t n, int64_t k, const uint8_t* packed,
                                         const uint8_t* scales, const float* global_scales,
                                         void* h, nvfp4_out_t out, uint32_t* d_status,
                                         void* workspace, size_t ws_bytes, void* stream);

/* Grouped GEMM whose rows are gathered through an index (routing-aware MoE
 * input, with no permuted copy of the activations): routed row r (rows in
 * expert order, segments as in nvfp4_grouped_gemm) computes with token row
 * x[row_index[r]] of x [x_rows][k]; y keeps the routed order.  act = 0 gives
 * y [rows][n] as nvfp4_grouped_gemm, act = 1 gives h [rows][n / 2] as
 * nvfp4_grouped_gemm_swiglu (same row-order requirement, n % 32 == 0).
 * row_index: device int32 [rows], 4-byte aligned; an index outside
 * [0, x_rows) sets NVFP4_DSTATUS_BAD_INDEX and that row computes as if its
 * activations were zero.  x_rows * k * 2 must fit in 32 bits (else
 * NVFP4_ERR_UNSUPPORTED).  Workspace: nvfp4_grouped_gemm_workspace_size(rows,
 * num_experts, n, k).  The gather is the routing-aware read of the fused MoE
 * layer ("The FP4 Frontier", Finding 5: one grouped GEMM over all experts). */
nvfp4_status_t nvfp4_grouped_gemm_gather(const void* x_bf16, int64_t x_rows,
                                         const int32_t* row_index, int64_t rows,
                                         const int32_t* expert_offsets, int64_t num_experts,
                                         int64_t n, int64_t k, const uint8_t* packed,
                                         const uint8_t* scales, const float* global_scales,
                                         void* y, nvfp4_out_t out, int32_t act,
                                         uint32_t* d_status, void* workspace, size_t ws_bytes,
                                         void* stream);

/* MoE MLP in one persistent launch ("The FP4 Frontier", Finding 5: fuse the
 * gate_up GEMM, SiLU and the down GEMM into a single persistent kernel):
 *   h = nvfp4_grouped_gemm_swiglu(x, up weights)      h [rows][d_ff]
 *   y = nvfp4_grouped_gemm(h, down weights)           y [rows][d_model]
 * over the same expert segments.  Neither product splits K here, so h and
 * y equal, bit for bit, what those two calls return when their schedules do
 * not split K either (the same kernels and summation order); a K split there
 * sums in another order, within the same error bound.  x [rows][d_model] holds
 * the routed rows sorted by expert; up_packed[e] [2 d_ff][d_model/2] (32-row
 * gate/up groups, as for nvfp4_grouped_gemm_swiglu), up_scales, up_global[e];
 * down_packed[e] [d_model][d_ff/2], down_scales, down_global[e].  h (caller-
 * allocated, written: BF16) is the intermediate; y gets `out`.
 * The launch's workgroups first compute every gate_up tile, then every down
 * tile; a down tile waits (a bounded poll of a per-row-tile count in the
 * workspace) until all gate_up tiles of its rows are stored.  The grid is
 * sized so that all workgroups are resident; should one wait time out anyway
 * (another kernel holding CUs), NVFP4_DSTATUS_WAIT_TIMEOUT is set, that
 * workgroup stops waiting, and y is unspecified.
 * Requirements: d_model % 64 == 0, d_ff % 64 == 0, 2 d_ff and d_model at most
 * 2^23, and a schedule in which both products take the same K-phase kernel
 * configuration; otherwise NVFP4_ERR_UNSUPPORTED and nothing is enqueued (the
 * two calls above then compute the result).  Workspace:
 * nvfp4_grouped_mlp_workspace_size() bytes; the call zeroes its per-row-tile
 * counts (after the first nvfp4_workspace_counter_bytes(), which it never
 * touches) on `stream`, so the buffer may also serve the GEMM calls.
 * Alignment, offsets and status as nvfp4_grouped_gemm. */
nvfp4_status_t nvfp4_grouped_mlp(const void* x_bf16, int64_t rows,
                                 const int32_t* expert_offsets, int64_t num_experts,
                                 int64_t d_model, int64_t d_ff, const uint8_t* up_packed,
                                 const uint8_t* up_scales, const float* up_global,
                                 const uint8_t* down_packed, const uint8_t* down_scales,
                                 const float* down_global, void* h, void* y, nvfp4_out_t out,
                                 uint32_t* d_status, void* workspace, size_t ws_bytes,
                                 void* stream);
size_t nvfp4_grouped_mlp_workspace_size(int64_t rows, int64_t num_experts, int64_t d_model,
                                        int64_t d_ff);
/* Name of the kernel instantiation nvfp4_grouped_mlp launches for this shape
 * ("" when the shape is not supported). */
const char* nvfp4_grouped_mlp_kernel_name(int64_t rows, int64_t num_experts, int64_t d_model,
                                          int64_t d_ff);

/* MoE combine, the scatter half of the routing-aware MoE layer ("The FP4
 * Frontier", Finding 5): out[t][c] = sum_j weights[t][j] * y[token_rows[t][j]][c]
 * for t < tokens, j < topk, summed in slot order in FP32 and rounded once
 * (RNE) for NVFP4_OUT_BF16.  y [rows][n] (y_type: BF16 or F32) holds the
 * routed rows, e.g. the down projection's output in expert order;
 * token_rows [tokens][topk] (device int32) names each token's routed rows, a
 * negative entry meaning an empty slot; weights [tokens][topk] (device FP32)
 * are the router weights.  out [tokens][n] (out_type).  No atomics: the
 * result is bitwise reproducible.  n must be a multiple of 8 and y, out
 * 16-byte aligned; token_rows and weights 4-byte aligned; 1 <= topk <= 64.
 * A row id >= rows sets NVFP4_DSTATUS_BAD_INDEX and that slot contributes
 * nothing.  tokens == 0 is a no-op.  No workspace. */
nvfp4_status_t nvfp4_moe_combine(const void* y, nvfp4_out_t y_type, int64_t rows,
                                 const int32_t* token_rows, const float* weights,
                                 int64_t tokens, int64_t topk, int64_t n, void* out,
                                 nvfp4_out_t out_type, uint32_t* d_status, void* stream);

/* W4A4: the activations are NVFP4 too, in the weights' encoding (block-scaled
 * FP4 data and scales for both operands: "The SM120 FP4 GEMM Kernel
 * Investigation", section "The Comprehensive Synthesis: Message 6").
 * x_packed [rows][k/2] and x_scales [rows][k/16] as written by nvfp4_quantize
 * for the activation tensor, x_global_scale one device float (its g).
 * y = x_global_scale * g[e] * x_dec . w_dec^T over each expert's rows, FP32
 * accumulation, x_dec / w_dec the decoded operands without their global
 * scales.  The activations are decoded once per call into the workspace
 * (BF16, exact), then the W4A16 kernels run on them with the global scale
 * product fl32(g[e] * x_global_scale); the workspace therefore always has a
 * nonzero size (nvfp4_*_w4a4_workspace_size) and must be initialised once
 * with nvfp4_workspace_init like the GEMM workspaces.  Its first
 * nvfp4_workspace_counter_bytes() bytes are the split-K counters and are
 * never used for the activations, so one workspace can serve W4A16 and W4A4
 * calls of any shape.  Same argument rules,
 * alignment and status behaviour as nvfp4_gemm / nvfp4_grouped_gemm
 * (x_packed takes the place of x_bf16); x_scales and x_global_scale must be
 * non-null, x_global_scale 4-byte aligned. */
nvfp4_status_t nvfp4_gemm_w4a4(const uint8_t* x_packed, const uint8_t* x_scales,
                               const float* x_global_scale, int64_t m, int64_t n, int64_t k,
                               const uint8_t* packed, const uint8_t* scales,
                               const float* global_scale, void* y, nvfp4_out_t out,
                               void* workspace, size_t ws_bytes, void* stream);
nvfp4_status_t nvfp4_grouped_gemm_w4a4(const uint8_t* x_packed, const uint8_t* x_scales,
                                       const float* x_global_scale, int64_t rows,
                                       const int32_t* expert_offsets, int64_t num_experts,
                                       int64_t n, int64_t k, const uint8_t* packed,
                                       const uint8_t* scales, const float* global_scales,
                                       void* y, nvfp4_out_t out, uint32_t* d_status,
                                       void* workspace, size_t ws_bytes, void* stream);
size_t nvfp4_gemm_w4a4_workspace_size(int64_t m, int64_t n, int64_t k);
size_t nvfp4_grouped_gemm_w4a4_workspace_size(int64_t rows, int64_t num_experts, int64_t n,
                                              int64_t k);

/* Dense W4A16 GEMM for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, result and error behaviour as
 * nvfp4_gemm (bit-identical output: the same schedule and kernels), without
 * the workspace: the split-K counters and partial tiles live in a scratch
 * array inside the library, one per GPU, of NVFP4_NOALLOC_SCRATCH_BYTES bytes
 * (64 KiB of counters + 16 MiB of partial tiles), held from the library's
 * load until the process ends.  A shape whose schedule needs more returns
 * NVFP4_ERR_UNSUPPORTED and enqueues nothing.  The call allocates nothing;
 * its first call on a device looks up that device's array and zeroes the
 * counter region with a fill kernel on `stream` (no memset node).  All calls
 * on one GPU share its array: calls that may overlap on one GPU (several
 * streams, or host threads) race and must be serialized by the caller. */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)65536 + ((size_t)16 << 20))
nvfp4_status_t nvfp4_gemm_noalloc(const void* x_bf16, int64_t m, int64_t n, int64_t k,
                                  const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scale, void* y, nvfp4_out_t out,
                                  void* stream);

/* Workspace sizes (bytes) for the calls above; 0 means none is needed.  The
 * sizes depend on the current device's compute-unit count. */
size_t nvfp4_quantize_workspace_size(int64_t batch, int64_t n, int64_t k);
size_t nvfp4_gemm_workspace_size(int64_t m, int64_t n, int64_t k);
size_t nvfp4_grouped_gemm_workspace_size(int64_t rows, int64_t num_experts, int64_t n,
                                         int64_t k);
/* Name of the kernel instantiation (as profilers print it, e.g.
 * "nvfp4::gemm_kp_kernel<64, 4, 8, 256, false>") that nvfp4_gemm (grouped = 0,
 * num_experts = 1) or nvfp4_grouped_gemm / _swiglu (grouped = 1; gather = 1:
 * nvfp4_grouped_gemm_gather) launches for this shape on the current device,
 * under the current tuning environment.  Static string; "" for an invalid
 * shape.  For reporting (per-kernel profiles, rooflines); it enqueues
 * nothing. */
const char* nvfp4_kernel_name(int64_t rows, int64_t num_experts, int64_t n, int64_t k,
                              int32_t grouped, int32_t gather);

/* Bytes at the start of any workspace that hold tile counters. */
size_t nvfp4_workspace_counter_bytes(void);

/* Zero the counter region of a workspace of ws_bytes bytes on `stream` (a
 * fill kernel, no memset node, so it may be captured in a HIP graph). */
nvfp4_status_t nvfp4_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* nvfp4_status_string(nvfp4_status_t status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int nvfp4_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H_ */
