// gemv.hip -- dense decode products: one to six token rows (gemv_kernel) and
// 7 to 64 rows (decode_sk_kernel); decode_mfma_kernel serves five and six
// rows whose K is too long to stage, and 7 to 16 rows when the split-K
// kernel is switched off or its counters would not hold the column tiles.
//
// One to six rows:
//
// Decode is the bandwidth-bound case ("The FP4 Frontier", Finding 7).  With
// so few rows a 16-row MFMA tile is mostly padding, and the in-register
// dequantization (16 VALU instructions per 8 weights) is what bounds the
// K-phase kernel.  Here the block scale leaves the inner loop instead; with
// the two scale tiers of "The Blackwell Architectural Split: NVFP4, Attention,
// and Consumer Silicon", section "Preserving precision" (an E4M3 factor per
// 16-element block, an FP32 factor per tensor):
//   y[m][n] = g * sum_b s[n][b] * (sum_{k in b} x[m][k] * e2m1(q[n][k]))
// The inner sum runs on the packed BF16 dot product: the FP4 convert turns
// two nibbles into two exact BF16 values (scale operand 1.0), and one
// v_dot2c_f32_bf16 multiplies them with two activations and adds both
// products into an FP32 accumulator.  That is about one VALU instruction per
// weight per row instead of two plus an MFMA share.
//
// Layout: one workgroup of 8 waves per 16 output columns.  Lane 4r + c of a
// wave reads row n0 + r; the four lanes of a row read four consecutive 16-byte
// chunks (32 weights each, 64 contiguous bytes), the waves take the row's
// next 128-byte groups in turn, so every chunk of the row is read once and
// each lane keeps up to kGemvBatch chunks in flight.  The token rows are
// staged in LDS once; their loads go out before the weights', so the staging
// waits for them alone and not for the weight stream behind them.  The
// partial sums are reduced in a fixed order: chunk order within a lane, the
// four lanes of a row, then the eight waves.
#include "nvfp4_internal.hpp"
#include "device_common.hpp"

namespace nvfp4 {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr int kGemvCols = 16;      // weight rows (output columns) per workgroup
constexpr int kGemvBatch = 8;      // chunks a lane loads before it multiplies them

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemv_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr uint32_t kGemvOffNone = 0x80000000u;  // beyond every resource: loads return 0

// Chunks c0, c0 + STRIDE, ... (kGemvBatch of them) of weight row r of the
// workgroup's 16 rows: 16 packed bytes and two scale bytes each.  Buffer
// loads with no branch: chunks past the row, and rows past N (past the
// resources), read as zero.
template <int STRIDE>
__device__ __forceinline__ void gemv_load_batch(uint4 (&pk)[kGemvBatch], uint32_t (&sc)[kGemvBatch],
                                                __amdgpu_buffer_rsrc_t rw,
                                                __amdgpu_buffer_rsrc_t rs, int r, int K, int c0,
                                                int C) {
#pragma unroll
  for (int b = 0; b < kGemvBatch; ++b) {
    const int c = c0 + STRIDE * b;
    const bool ok = c < C;
    const uint32_t wo = ok ? (uint32_t)(r * (K / 2) + 16 * c) : kGemvOffNone;
    const uint32_t so = ok ? (uint32_t)(r * (K / 16) + 2 * c) : kGemvOffNone;
    pk[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0));
    sc[b] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
  }
}

template <int M>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xl[];  // [M][K] bf16
  __shared__ float red[kGemvWaves][M][kGemvCols];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.k, N = p.n;
  const int n0 = blockIdx.x * kGemvCols;
  const int r = lane >> 2, cl = lane & 3;
  const int C = K / 32;  // 32-weight chunks per row
  constexpr int kStride = 4 * kGemvWaves;  // chunks between a lane's consecutive chunks
  const int rows16 = min(kGemvCols, N - n0);
  const __amdgpu_buffer_rsrc_t rw = gemv_rsrc(p.w + (int64_t)n0 * (K / 2), (uint32_t)(rows16 * (K / 2)));
  const __amdgpu_buffer_rsrc_t rs = gemv_rsrc(p.s + (int64_t)n0 * (K / 16), (uint32_t)(rows16 * (K / 16)));
  uint4 pk[kGemvBatch];
  uint32_t sc[kGemvBatch];
  // the token rows go out first (registers, then LDS), then the first weight
  // batch: the staging then waits for the token rows only, not for the
  // weights behind them
  constexpr int kXV = (int)(kGemvMaxXBytes / 16 / kGemvThreads);  // 16-byte vectors per thread
  const int nv = M * K / 8;
  const __amdgpu_buffer_rsrc_t rx = gemv_rsrc(p.x, (uint32_t)nv * 16u);
  uint4 xv[kXV];
#pragma unroll
  for (int i = 0; i < kXV; ++i) {
    const int idx = tid + i * kGemvThreads;
    xv[i] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, idx < nv ? (uint32_t)idx * 16u : kGemvOffNone,
                                                     0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);
  int c0 = 4 * wave + cl;
  gemv_load_batch<kStride>(pk, sc, rw, rs, r, K, c0, C);
  __builtin_amdgcn_sched_barrier(0);
  {
    uint4* dst = reinterpret_cast<uint4*>(xl);
#pragma unroll
    for (int i = 0; i < kXV; ++i) {
      const int idx = tid + i * kGemvThreads;
      if (idx < nv) dst[idx] = xv[i];
    }
  }
  __syncthreads();
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  for (; c0 < C; c0 += kStride * kGemvBatch) {
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int c = c0 + kStride * b;
      if (c < C) {
        // the chunk's two blocks: dwords 0-1 and 2-3, scale bytes 0 and 1
        const float s0 = decode_e4m3<0>(sc[b]), s1 = decode_e4m3<1>(sc[b]);
        const uint32_t pw[4] = {pk[b].x, pk[b].y, pk[b].z, pk[b].w};
        bf16x2_t q[16];  // q[4 j + t]: weights 8 j + 2 t and 8 j + 2 t + 1 of the chunk
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          q[4 * j + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pw[j], 1.0f, 0);
          q[4 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pw[j], 1.0f, 1);
          q[4 * j + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pw[j], 1.0f, 2);
          q[4 * j + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pw[j], 1.0f, 3);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint4* xr = reinterpret_cast<const uint4*>(xl + m * K + 32 * c);
          float part[2] = {0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint4 xv = xr[j];  // activations 8 j .. 8 j + 7 of the chunk
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int t = 0; t < 4; ++t)
              part[j >> 1] = __builtin_amdgcn_fdot2_f32_bf16(
                  q[4 * j + t], __builtin_bit_cast(bf16x2_t, xw[t]), part[j >> 1], false);
          }
          acc[m] += s0 * part[0];
          acc[m] += s1 * part[1];
        }
      }
    }
    if (c0 + kStride * kGemvBatch < C)
      gemv_load_batch<kStride>(pk, sc, rw, rs, r, K, c0 + kStride * kGemvBatch, C);
  }
  // the four lanes of a row, then the waves, in a fixed order
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = acc[m];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    if (cl == 0) red[wave][m][r] = v;
  }
  __syncthreads();
  if (tid < M * kGemvCols) {
    const int m = tid / kGemvCols, rr = tid % kGemvCols;
    const int col = n0 + rr;
    if (col < N) {
      float sum = red[0][m][rr];
#pragma unroll
      for (int w = 1; w < kGemvWaves; ++w) sum += red[w][m][rr];
      const float v = p.g[0] * sum;
      const int64_t o = (int64_t)m * N + col;
      if (p.out_f32)
        static_cast<float*>(p.y)[o] = v;
      else
        static_cast<uint16_t*>(p.y)[o] = (uint16_t)float_to_bf16_rne(v);
    }
  }
}

// ---- one MFMA row tile, whole K per workgroup (up to 16 rows) -----------------
//
// With many rows the per-row dot products cost more than one BF16 MFMA row
// tile, but the K-phase kernel's latency structure (a ring of 128-deep stages,
// split K with a partial-tile hand-off) still dominates at decode sizes.  This
// kernel keeps every load of a workgroup in flight at once instead: one
// workgroup of 8 waves per 16 output columns, whole K; wave w takes the
// 128-deep K groups j = w, w + 8, ...  Within a group, lane (n, g) = (l % 16,
// l / 16) loads 16 contiguous bytes of weight row n (K = 128 j + 32 g .. + 31),
// their two scale bytes, and the matching 64 activation bytes of token row
// l % 16 straight from global memory (the token rows are read by every
// workgroup and stay in L2).  The MFMA's 32 K slots are a permutation of real
// K -- slot 8 g + i of step t is K = 128 j + 32 g + 8 t + i -- applied to both
// operands alike, so the product is unchanged.  Partial tiles of the 8 waves
// are summed in wave order through LDS.
// JB: 128-deep K groups a lane loads before it multiplies them (1 to 8; the
// launch picks the smallest count that covers a wave's groups in one pass
// when it can).
template <int JB>
__global__ __launch_bounds__(kGemvThreads) void decode_mfma_kernel(GemmParams p) {
  __shared__ f32x4_t red[kGemvWaves][kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.k, N = p.n, M = (int)p.rows;
  const int n0 = blockIdx.x * kGemvCols;
  const int c16 = lane & 15, g = lane >> 4;
  const int n = n0 + c16;
  const bool col_ok = n < N, row_ok = c16 < M;
  const int J = K / 128;
  const uint8_t* wrow = p.w + (int64_t)(col_ok ? n : 0) * (K / 2) + 16 * g;
  const uint8_t* srow = p.s + (int64_t)(col_ok ? n : 0) * (K / 16) + 2 * g;
  const uint16_t* xrow = p.x + (int64_t)(row_ok ? c16 : 0) * K + 32 * g;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int j0 = wave; j0 < J; j0 += kGemvWaves * JB) {
    uint4 wv[JB];
    uint32_t sv[JB];
    bf16x8_t xv[JB][4];
    // unconditional loads, so that no branch separates them and each group
    // is multiplied as soon as its own loads have landed: a group past K
    // re-reads the last group (and is not multiplied), a column past N reads
    // weight row 0 and a token row past M reads token row 0 (their outputs
    // are not stored)
#pragma unroll
    for (int b = 0; b < JB; ++b) {
      const int j = min(j0 + kGemvWaves * b, J - 1);
      wv[b] = *reinterpret_cast<const uint4*>(wrow + 64 * (int64_t)j);
      sv[b] = *reinterpret_cast<const uint16_t*>(srow + 8 * (int64_t)j);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        xv[b][t] = *reinterpret_cast<const bf16x8_t*>(xrow + 128 * (int64_t)j + 8 * t);
    }
#pragma unroll
    for (int b = 0; b < JB; ++b) {
      const int j = j0 + kGemvWaves * b;
      if (j < J) {  // wave-uniform
        const float s0 = decode_e4m3<0>(sv[b]), s1 = decode_e4m3<1>(sv[b]);
        const uint32_t pw[4] = {wv[b].x, wv[b].y, wv[b].z, wv[b].w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[b][t], dequant8(pw[t], t < 2 ? s0 : s1),
                                                        acc, 0, 0, 0);
      }
    }
  }
  // lane l holds rows 4 (l / 16) .. + 3 of column l % 16
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < kGemvWaves; ++w) sum += red[w][lane];
    const float gv = p.g[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M && col_ok) {
        const float v = gv * sum[i];
        const int64_t o = (int64_t)m * N + n;
        if (p.out_f32)
          static_cast<float*>(p.y)[o] = v;
        else
          static_cast<uint16_t*>(p.y)[o] = (uint16_t)float_to_bf16_rne(v);
      }
    }
  }
}

// ---- 7 to 64 rows: split K, a workgroup's whole weight share in flight --------
//
// Decode moves each weight byte once, and with a few dozen rows the per-CU
// weight share is a few tens of KB: the time is about one HBM latency plus
// the transfer, provided every load of the share is in flight from the start.
// The K-phase kernel's ring keeps only a few 128-deep stages in flight, and
// decode_mfma_kernel reads the token rows once per 16 columns (at 64 rows the
// activations would outweigh the weights 16:1).  Here a unit is 64 output
// columns x one K split (k_split, at most 16 groups of 128), with the split
// count chosen so that the units about fill the CUs (N = 4096, K = 7168: 64
// column tiles x 4 splits).  Wave w of the 8 owns the unit's 128-deep K groups
// j with j % 8 == w, for all four 16-column tiles, so every activation
// fragment it reads from LDS feeds four MFMAs.  Only wave w reads the token
// rows of its groups, so they go straight from memory (buffer_load ... lds)
// into a region of LDS of its own, and each wave waits for its own loads
// only: no barrier stands between the loads and the MFMAs.  Each wave first
// issues the token rows of its first group (of both, when 8 waves x 2 groups
// fit the LDS, up to 32 rows), then every weight load of its share -- per
// group and column tile 16 bytes of its weight row at K = 128 j + 32 (l / 16)
// and the two scale bytes, the K-slot permutation of decode_mfma_kernel.
// With more rows its second group's token rows replace the first's once that
// group is multiplied out.  A row's 16-byte chunk c sits at c ^ (row % 16).
// (Staged through registers into one shared LDS tile in phases of groups,
// with a barrier per phase, the launch took 6-10 % longer at 16-64 rows.)
// The waves' sums meet through LDS in a fixed order, the splits of a column
// tile through device-scope partial tiles and an arrival counter, and the
// last split sums them in split order (so the result does not depend on
// timing).
constexpr int kDskXBytes = 128 * 1024;  // LDS for the waves' token-row regions
// groups a wave's region holds: both of its groups when they fit, else one
template <int NF>
constexpr int kDskRes = kGemvWaves * (kDskMaxGroups / kGemvWaves) * NF * 4096 <= kDskXBytes
                            ? kDskMaxGroups / kGemvWaves
                            : 1;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dsk_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// device-scope (sc1) buffer accesses: past the non-coherent L2
constexpr int kDskCpol = 16;
constexpr uint32_t kDskOffNone = 0x80000000u;  // beyond every resource: loads return 0

template <int NF>
__global__ __launch_bounds__(kGemvThreads) void decode_sk_kernel(GemmParams p) {
  constexpr int BM = NF * 16;
  constexpr int CT = kDskCols / 16;                  // column tiles per unit
  constexpr int GPW = kDskMaxGroups / kGemvWaves;    // groups per wave (upper bound)
  constexpr int RES = kDskRes<NF>;                   // groups a wave's region holds
  constexpr int GB = BM * 256;                       // bytes of one group's token rows
  constexpr int XL = GB / 1024;                      // 1 KB loads per group
  static_assert(kDskCols % 16 == 0 && kDskMaxGroups % kGemvWaves == 0, "unit shape");
  static_assert(GPW == 2 && (RES == 1 || RES == GPW), "a wave's groups: one or both resident");
  // a group's rows are whole 1 KB loads (four 256-byte rows each), and the
  // waves' regions (RES groups each) fit the LDS set aside for them
  static_assert(XL * 1024 == GB && BM % 4 == 0, "group rows per load");
  static_assert(kGemvWaves * RES * GB <= kDskXBytes, "token-row regions fit");
  __shared__ __attribute__((aligned(16))) uint8_t xs[kGemvWaves * RES * GB];
  __shared__ int last_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int K = p.k, N = p.n, M = (int)p.rows;
  // unit: XCD-major placement (workgroup b runs on XCD b % 8), so the column
  // tiles of one split -- which read the same token-row range -- share an L2
  const int G = gridDim.x, b = blockIdx.x;
  const int v = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int s = v / p.n_tiles, nt = v % p.n_tiles;
  const int k0 = s * p.k_split;
  const int ng = (min(K, k0 + p.k_split) - k0) / 128;  // K groups of this unit
  const int nrows = min(kDskCols, N - nt * kDskCols);  // weight rows of the unit
  // buffer resources: loads past a resource (rows past N, rows past M, K
  // groups past the unit) read zero, so no load sits behind a branch
  const u32x4_t rxw = rsrc_words(p.x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rw =
      dsk_rsrc(p.w + (int64_t)nt * kDskCols * (K / 2), (uint32_t)(nrows * (K / 2)));
  const __amdgpu_buffer_rsrc_t rs =
      dsk_rsrc(p.s + (int64_t)nt * kDskCols * (K / 16), (uint32_t)(nrows * (K / 16)));

  // The token rows of group j (all BM rows, 256 bytes each) into slot `sl`
  // of this wave's region, straight from memory (buffer_load ... lds): load t
  // covers rows 4t .. 4t + 3, and the 16-byte piece at position q of row r
  // holds chunk q ^ (r % 16) of the row.  Rows past M and groups past the
  // unit load zeros.
  uint8_t* const region = xs + wave * (RES * GB);
  auto load_group = [&](int j, int sl) {
    const uint32_t dst = lds_addr(region + sl * GB);
#pragma unroll
    for (int t = 0; t < XL; ++t) {
      const int r = 4 * t + (lane >> 4), q = lane & 15;
      const int c = q ^ (r & 15);
      const uint32_t off = (r < M && j < ng)
                               ? ((uint32_t)r * (uint32_t)K + (uint32_t)(k0 + 128 * j + 8 * c)) * 2u
                               : kDskOffNone;
      lds_dma16(dst + t * 1024, off, 0u, rxw);
    }
  };

  // The wave's first group (both, when they fit) goes out before the weights
  // (a scheduling fence: no memory fence, which would make the compiler wait
  // for the loads).
  load_group(wave, 0);
  if constexpr (RES == GPW) load_group(wave + kGemvWaves, 1);
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t wv[GPW][CT];
  uint32_t sv[GPW][CT];
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int j = wave + kGemvWaves * i;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int r = 16 * ct + c16;  // weight row within the unit
      const bool ok = j < ng;
      const uint32_t wo = ok ? (uint32_t)(r * (K / 2) + (k0 + 128 * j) / 2 + 16 * g) : kDskOffNone;
      const uint32_t so = ok ? (uint32_t)(r * (K / 16) + (k0 + 128 * j) / 16 + 2 * g) : kDskOffNone;
      wv[i][ct] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0));
      sv[i][ct] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  f32x4_t acc[NF][CT];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[f][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // step t of group i with its A fragments and the group's weights
  auto mma_step = [&](int i, int t, const bf16x8_t (&a)[NF]) {
    bf16x8_t bq[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float sc = t < 2 ? decode_e4m3<0>(sv[i][ct]) : decode_e4m3<1>(sv[i][ct]);
      bq[ct] = dequant8(wv[i][ct][t], sc);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        acc[f][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f], bq[ct], acc[f][ct], 0, 0, 0);
  };
  // multiply out group i of this wave (token rows in region slot sl)
  auto group = [&](int i, int sl) {
    const uint8_t* xg = region + sl * GB;
    // A fragments of step t + 1 are read while step t is dequantized and
    // multiplied (LDS latency behind the MFMAs)
    bf16x8_t a[2][NF];
    auto read_a = [&](bf16x8_t (&dst)[NF], int t) {
      const int c = 4 * g + t;  // K = 128 j + 32 g + 8 t .. + 7
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int row = 16 * f + c16;
        dst[f] = *reinterpret_cast<const bf16x8_t*>(xg + (row * 16 + (c ^ (row & 15))) * 16);
      }
    };
    read_a(a[0], 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < 3) read_a(a[(t + 1) & 1], t + 1);
      mma_step(i, t, a[t & 1]);
    }
  };
  // Only this wave reads its region, so it waits for its own loads alone:
  // after the first group's token rows come the second group's (when both
  // are resident) and the 2 CT weight and scale loads of each group.
  constexpr int kWLoads = GPW * CT * 2;
  if constexpr (RES == GPW) {
    if (wave < ng) {  // wave-uniform
      wait_vmcnt_c<XL + kWLoads>();
      group(0, 0);
    }
    if (wave + kGemvWaves < ng) {
      wait_vmcnt_c<kWLoads>();
      group(1, 1);
    }
  } else if (wave < ng) {
    wait_vmcnt_c<kWLoads>();
    group(0, 0);
    if (wave + kGemvWaves < ng) {
      // the second group replaces the first in the region, once this wave's
      // reads of it are done (holding all of the first group's fragments in
      // registers, to load the second one sooner, spills at 48 and 64 rows)
      wait_lgkmcnt0();
      load_group(wave + kGemvWaves, 0);
      wait_vmcnt_c<0>();
      group(1, 0);
    }
  }

  // every token-row load of this wave has landed (those of groups past the
  // unit write zeros) before the regions are reused below
  wait_vmcnt_c<0>();

  // Sum the waves in a fixed order, (((w0 + w4) + (w1 + w5)) + (w2 + w6)) +
  // (w3 + w7): each wave publishes its sums at the start of its own region
  // (which no other wave reads, so it needs no barrier first), and after one
  // barrier every thread adds the eight, in that order, for its share of the
  // tile (float4 q = (f CT + ct) 64 + lane of the accumulator layout) -- all
  // 512 threads at once, not one wave.
  constexpr int Q = NF * CT * kWave;                            // float4 values per tile
  constexpr int QPT = (Q + kGemvThreads - 1) / kGemvThreads;    // per thread: 1 or 2
  static_assert(Q * 16 <= RES * GB, "a wave's sums fit its region");
  auto slot = [&](int w) { return reinterpret_cast<f32x4_t*>(xs + w * (RES * GB)); };
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) slot(wave)[(f * CT + ct) * kWave + lane] = acc[f][ct];
  __syncthreads();
  f32x4_t sum[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int q = tid + i * kGemvThreads;
    if (q < Q)
      sum[i] = (((slot(0)[q] + slot(4)[q]) + (slot(1)[q] + slot(5)[q])) +
                (slot(2)[q] + slot(6)[q])) +
               (slot(3)[q] + slot(7)[q]);
  }
  // float4 q of the accumulator layout -> its 4 elements of the row-major
  // FP32 tile in LDS (rows 16 f + 4 g + r, column 16 ct + l % 16)
  float* tile = reinterpret_cast<float*>(xs);  // [BM][kDskCols]
  const float gv = p.g[0];
  auto to_tile = [&](int q, const f32x4_t& v) {
    const int slot = q / kWave, l = q % kWave;
    const int f = slot / CT, ct = slot % CT;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      tile[(16 * f + 4 * (l >> 4) + r) * kDskCols + 16 * ct + (l & 15)] = gv * v[r];
  };
  const int S = p.splits;
  if (S > 1) {
    // every thread stores its share of the partial tile (device-scope
    // stores), waits for them, and one thread counts the arrival
    const __amdgpu_buffer_rsrc_t part =
        dsk_rsrc(p.partials + (int64_t)nt * S * (BM * kDskCols), (uint32_t)(S * BM * kDskCols * 4));
    auto poff = [&](int ss, int q) { return (uint32_t)((ss * (BM * kDskCols) + 4 * q) * 4); };
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = tid + i * kGemvThreads;
      if (q < Q)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, sum[i]), part,
                                               poff(s, q), 0, kDskCpol);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the partial stores have completed
    __syncthreads();
    if (tid == 0) {
      const uint32_t old =
          __hip_atomic_fetch_add(&p.counters[nt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = old == (uint32_t)(S - 1);
    }
    __syncthreads();
    if (!last_flag) return;  // uniform: another split finishes the tile
    // The last split sums all S partial tiles (its own included, as stored)
    // in split order, each thread for its share; the loads of up to U splits
    // of all its shares are in flight before it adds any, so the hand-off
    // costs one memory latency per U splits.
    constexpr int U = 8;
    f32x4_t tot[QPT];
    for (int s0 = 0; s0 < S; s0 += U) {
      f32x4_t v[QPT][U];
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const int q = tid + i * kGemvThreads;
#pragma unroll
        for (int u = 0; u < U; ++u)
          v[i][u] = __builtin_bit_cast(
              f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                           part, (q < Q && s0 + u < S) ? poff(s0 + u, q) : kDskOffNone, 0, kDskCpol));
      }
#pragma unroll
      for (int i = 0; i < QPT; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (s0 + u < S) tot[i] = (s0 + u == 0) ? v[i][u] : tot[i] + v[i][u];
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = tid + i * kGemvThreads;
      if (q < Q) to_tile(q, tot[i]);
    }
    if (tid == 0) __hip_atomic_store(&p.counters[nt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    __syncthreads();  // every exchange read is done: the tile may overwrite the slots
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = tid + i * kGemvThreads;
      if (q < Q) to_tile(q, sum[i]);
    }
  }
  // Output: the tile is row-major in LDS (FP32, g applied); every thread
  // writes whole 16-byte pieces of the tile's rows -- one store per piece
  // instead of one 2- or 4-byte store per element -- and only the pieces
  // that reach past column N, or whose rows are not 16-byte aligned, go
  // element by element.
  __syncthreads();
  const int esz = p.out_f32 ? 4 : 2;
  const int cpr = kDskCols * esz / 16;  // 16-byte pieces per tile row
  const int ncol0 = nt * kDskCols;
  const bool rows_aligned = (N * esz) % 16 == 0;
  const __amdgpu_buffer_rsrc_t ry = dsk_rsrc(p.y, (uint32_t)M * (uint32_t)N * (uint32_t)esz);
  for (int q = tid; q < BM * cpr; q += kGemvThreads) {
    const int row = q / cpr, piece = q % cpr;
    if (row >= M) continue;
    const int per = 16 / esz;                // elements per piece
    const int col = ncol0 + piece * per;     // first column of the piece
    const float* src = tile + row * kDskCols + piece * per;
    const uint32_t base = ((uint32_t)row * (uint32_t)N + (uint32_t)col) * (uint32_t)esz;
    if (rows_aligned && col + per <= N) {
      u32x4_t v;
      if (p.out_f32) {
        v = u32x4_t{__float_as_uint(src[0]), __float_as_uint(src[1]), __float_as_uint(src[2]),
                    __float_as_uint(src[3])};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = float_to_bf16_rne(src[2 * e]) | (float_to_bf16_rne(src[2 * e + 1]) << 16);
      }
      __builtin_amdgcn_raw_buffer_store_b128(v, ry, base, 0, 0);
    } else {
      for (int e = 0; e < per; ++e) {
        if (col + e >= N) break;
        if (p.out_f32)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(src[e]), ry, base + 4u * e, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)float_to_bf16_rne(src[e]), ry,
                                                base + 2u * e, 0, 0);
      }
    }
  }
}

hipError_t launch_gemv(const GemmPlan& pl, const GemmParams& p, hipStream_t stream) {
  if (pl.kind == 8) {
    const dim3 grid((unsigned)pl.grid), block(kGemvThreads);
    switch (pl.bm) {
      case 16: hipLaunchKernelGGL(decode_sk_kernel<1>, grid, block, 0, stream, p); break;
      case 32: hipLaunchKernelGGL(decode_sk_kernel<2>, grid, block, 0, stream, p); break;
      case 48: hipLaunchKernelGGL(decode_sk_kernel<3>, grid, block, 0, stream, p); break;
      case 64: hipLaunchKernelGGL(decode_sk_kernel<4>, grid, block, 0, stream, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (pl.kind == 7) {
    const dim3 grid((unsigned)pl.grid), block(kGemvThreads);
    const int per_wave = (p.k / 128 + kGemvWaves - 1) / kGemvWaves;  // K groups per wave
    switch (per_wave < 8 ? per_wave : 8) {
      case 1: hipLaunchKernelGGL(decode_mfma_kernel<1>, grid, block, 0, stream, p); break;
      case 2: hipLaunchKernelGGL(decode_mfma_kernel<2>, grid, block, 0, stream, p); break;
      case 3: hipLaunchKernelGGL(decode_mfma_kernel<3>, grid, block, 0, stream, p); break;
      case 4: hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, block, 0, stream, p); break;
      case 5: hipLaunchKernelGGL(decode_mfma_kernel<5>, grid, block, 0, stream, p); break;
      case 6: hipLaunchKernelGGL(decode_mfma_kernel<6>, grid, block, 0, stream, p); break;
      case 7: hipLaunchKernelGGL(decode_mfma_kernel<7>, grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL(decode_mfma_kernel<8>, grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)pl.grid), block(kGemvThreads);
  switch (pl.bm) {
    case 1: hipLaunchKernelGGL(gemv_kernel<1>, grid, block, pl.dyn_lds, stream, p); break;
    case 2: hipLaunchKernelGGL(gemv_kernel<2>, grid, block, pl.dyn_lds, stream, p); break;
    case 3: hipLaunchKernelGGL(gemv_kernel<3>, grid, block, pl.dyn_lds, stream, p); break;
    case 4: hipLaunchKernelGGL(gemv_kernel<4>, grid, block, pl.dyn_lds, stream, p); break;
    case 5: hipLaunchKernelGGL(gemv_kernel<5>, grid, block, pl.dyn_lds, stream, p); break;
    case 6: hipLaunchKernelGGL(gemv_kernel<6>, grid, block, pl.dyn_lds, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
