// gemm.hip -- NVFP4 weight x BF16 activation GEMM (dense and MoE grouped)
// for gfx950.
//
// The method: weights are E2M1 nibbles with one E4M3 scale per 16 values
// along K and one FP32 scale per tensor ("The Blackwell Architectural Split:
// NVFP4, Attention, and Consumer Silicon", section "Preserving precision --
// dual-tier scale handling"); activations stay BF16 ("The SM120 FP4 GEMM
// Kernel Investigation", section "The Context").  At 16-64 tokens per expert
// the product is bound by memory bandwidth ("The FP4 Frontier", Finding 7),
// and the recommended schedule is one grouped, persistent kernel over all
// experts with smaller tiles and adaptive grids for small batches (same page,
// Finding 5).  Dequantization happens in registers, 16 values per scale, just
// before the matrix instruction -- the register-level idea of the A4Q section
// of the first page -- instead of staging unpacked weights in shared memory,
// which is what overflowed shared memory on the pages' hardware ("The
// Problem Shared Memory Brick Wall" on the same page).
//
// gfx950 design
//  - One persistent grid.  A work unit is (expert, row tile of BM rows,
//    column tile of 256 weight rows, K split).  Every workgroup reads the
//    expert offsets from device memory, builds the per-expert unit prefix in
//    LDS and walks units blockIdx.x, +gridDim.x, ...  Empty experts own no
//    units.  There is no host synchronization and no inter-workgroup wait.
//  - 4 waves per workgroup; each wave owns 64 weight rows = 4 MFMA column
//    tiles.  Lane l of a wave covers weight row (l % 16) of each tile and the
//    64-wide K range 64*(l/16) of every 256-wide K chunk: two 16-byte loads of
//    packed nibbles and one 4-byte load of its four block scales.  Each weight
//    byte is loaded from HBM once per row tile.
//  - MFMA v_mfma_f32_16x16x32_bf16.  Its 32 K slots are assigned so that lane
//    group q = l/16 supplies K = kc + 64q + 8i .. +7 in step i (i = 0..7) for
//    both operands; the order of a sum does not change its exact value, and
//    the assignment keeps every lane's weight bytes contiguous.
//  - Activations: a BM x 256 BF16 chunk is staged in LDS (rows padded by
//    16 bytes so the 16-byte fragment reads of 16 rows hit distinct banks)
//    and shared by the 4 waves.
//  - Dequant: a nibble pair becomes two exact FP32 values with the gfx950 FP4
//    conversion, is multiplied by the decoded E4M3 scale (exact), and the
//    upper halves form two BF16 values.  The global scale g is applied once
//    to the FP32 accumulator in the epilogue.
//  - Split-K (used when there are too few output tiles to fill the chip):
//    each split writes its FP32 partial tile to the workspace, bumps the
//    tile's counter, and the last arrival sums the partials in split order
//    (bitwise reproducible), resets the counter and writes the output.
#include <algorithm>
#include <cstdlib>

#include "device_common.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

constexpr int kNW = 4;                 // MFMA column tiles per wave
constexpr int kLdsStride = kKC + 8;    // BF16 elements per staged activation row

// Exclusive scan of one int per thread over the workgroup (256 threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kGemmThreads / kWave; ++w) {
    base += (w < wave) ? tmp[w] : 0;
    sum += tmp[w];
  }
  __syncthreads();
  *total = sum;
  return base + incl - v;
}

template <int BM, bool FAST>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmParams p) {
  constexpr int NF = BM / 16;  // MFMA row fragments
  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * kLdsStride];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_units[kMaxExperts + 1];
  __shared__ int s_tiles[kMaxExperts + 1];
  __shared__ int s_tmp[kGemmThreads / kWave];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;      // lane group: K sub-range of the chunk
  const int r16 = lane & 15;    // row within an MFMA tile
  const int E = p.num_experts;
  const int N = p.n;
  const int K = p.k;
  const int S = p.splits;

  // ---- expert segments and the unit prefix --------------------------------
  for (int e = tid; e <= E; e += kGemmThreads)
    s_off[e] = p.offsets ? p.offsets[e] : (e == 0 ? 0 : (int)p.rows);
  __syncthreads();
  int bad = 0;
  for (int e = tid; e < E; e += kGemmThreads) bad |= (s_off[e + 1] < s_off[e]);
  if (tid == 0) bad |= (s_off[0] != 0) | ((int64_t)s_off[E] != p.rows);
  bad = __syncthreads_or(bad);
  if (bad) {
    if (blockIdx.x == 0 && tid == 0 && p.d_status != nullptr)
      atomicOr(p.d_status, NVFP4_DSTATUS_BAD_OFFSETS);
    return;
  }
  // each thread owns experts [4*tid, 4*tid+4)
  int my_units = 0, my_tiles = 0;
  for (int e = 4 * tid; e < 4 * tid + 4 && e < E; ++e) {
    const int mt = (s_off[e + 1] - s_off[e] + BM - 1) / BM;
    my_tiles += mt * p.n_tiles;
    my_units += mt * p.n_tiles * S;
  }
  int total_units, total_tiles;
  int ubase = block_exclusive_scan(my_units, s_tmp, &total_units);
  int tbase = block_exclusive_scan(my_tiles, s_tmp, &total_tiles);
  for (int e = 4 * tid; e < 4 * tid + 4 && e < E; ++e) {
    s_units[e] = ubase;
    s_tiles[e] = tbase;
    const int mt = (s_off[e + 1] - s_off[e] + BM - 1) / BM;
    ubase += mt * p.n_tiles * S;
    tbase += mt * p.n_tiles;
  }
  if (tid == 0) {
    s_units[E] = total_units;
    s_tiles[E] = total_tiles;
  }
  __syncthreads();

  // ---- persistent loop over work units ------------------------------------
  for (int unit = blockIdx.x; unit < total_units; unit += gridDim.x) {
    // expert: last e with s_units[e] <= unit (empty experts have equal bounds)
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_units[mid] <= unit) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int seg0 = s_off[e], seg1 = s_off[e + 1];
    const int mtiles = (seg1 - seg0 + BM - 1) / BM;
    const int local = unit - s_units[e];
    const int mt = local % mtiles;
    const int rest = local / mtiles;
    const int ks = rest % S;
    const int nt = rest / S;
    const int tile = s_tiles[e] + nt * mtiles + mt;
    const int row0 = seg0 + mt * BM;
    const int row_end = min(row0 + BM, seg1);
    const int k_beg = ks * p.k_split;
    const int k_end = min(K, k_beg + p.k_split);

    const uint8_t* __restrict__ We = p.w + (int64_t)e * N * (K / 2);
    const uint8_t* __restrict__ Se = p.s + (int64_t)e * N * (K / 16);

    int nrow[kNW];
#pragma unroll
    for (int j = 0; j < kNW; ++j) nrow[j] = nt * kBN + wave * (kNW * 16) + j * 16 + r16;

    f32x4_t acc[NF][kNW];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < kNW; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int kc = k_beg; kc < k_end; kc += kKC) {
      // -- this lane's packed weights and scales for the chunk
      uint32_t wreg[kNW][8];
      uint32_t sreg[kNW];
      const int kpos = kc + 64 * q;
#pragma unroll
      for (int j = 0; j < kNW; ++j) {
        const bool rv = nrow[j] < N;
        if (FAST) {
          if (rv && kpos < k_end) {
            const u32x4_t* src =
                reinterpret_cast<const u32x4_t*>(We + (int64_t)nrow[j] * (K / 2) + kpos / 2);
            const u32x4_t a = __builtin_nontemporal_load(src);
            const u32x4_t b = __builtin_nontemporal_load(src + 1);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              wreg[j][t] = a[t];
              wreg[j][4 + t] = b[t];
            }
            sreg[j] = *reinterpret_cast<const uint32_t*>(Se + (int64_t)nrow[j] * (K / 16) +
                                                         kpos / 16);
          } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) wreg[j][t] = 0u;
            sreg[j] = 0u;
          }
        } else {
          uint32_t sv = 0u;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int kd = kpos + 8 * t;
            wreg[j][t] = (rv && kd < k_end)
                             ? *reinterpret_cast<const uint32_t*>(
                                   We + (int64_t)nrow[j] * (K / 2) + kd / 2)
                             : 0u;
          }
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int kb = kpos + 16 * b;
            const uint32_t byte =
                (rv && kb < k_end) ? (uint32_t)Se[(int64_t)nrow[j] * (K / 16) + kb / 16] : 0u;
            sv |= byte << (8 * b);
          }
          sreg[j] = sv;
        }
      }

      // -- stage the activation chunk [row0, row0+BM) x [kc, kc+256) in LDS
#pragma unroll
      for (int pass = 0; pass < BM / 8; ++pass) {
        const int pc = tid + kGemmThreads * pass;
        const int r = pc >> 5;
        const int c8 = (pc & 31) * 8;
        const int grow = row0 + r;
        const int kk = kc + c8;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (grow < row_end && kk < k_end)
          v = *reinterpret_cast<const u32x4_t*>(p.x + (int64_t)grow * K + kk);
        *reinterpret_cast<u32x4_t*>(&xs[r * kLdsStride + c8]) = v;
      }
      __syncthreads();

      // -- 8 MFMA steps of 32 K slots
      float sc[kNW][4];
#pragma unroll
      for (int j = 0; j < kNW; ++j) {
        sc[j][0] = decode_e4m3<0>(sreg[j]);
        sc[j][1] = decode_e4m3<1>(sreg[j]);
        sc[j][2] = decode_e4m3<2>(sreg[j]);
        sc[j][3] = decode_e4m3<3>(sreg[j]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bf16x8_t a[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f)
          a[f] = *reinterpret_cast<const bf16x8_t*>(
              &xs[(f * 16 + r16) * kLdsStride + 64 * q + 8 * i]);
#pragma unroll
        for (int j = 0; j < kNW; ++j) {
          const bf16x8_t b = dequant8(wreg[j][i], sc[j][i >> 1]);
#pragma unroll
          for (int f = 0; f < NF; ++f)
            acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f], b, acc[f][j], 0, 0, 0);
        }
      }
      __syncthreads();
    }

    // ---- split-K hand-off --------------------------------------------------
    if (S > 1) {
      float* part = p.partials + (int64_t)tile * S * (BM * kBN);
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < kNW; ++j)
          *reinterpret_cast<f32x4_t*>(part + (int64_t)ks * (BM * kBN) +
                                      (((wave * NF + f) * kNW + j) * kWave + lane) * 4) =
              acc[f][j];
      fence_release_agent();
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = atomicAdd(&p.counters[tile], 1u);
        s_flag = (old == (uint32_t)(S - 1));
      }
      __syncthreads();
      if (!s_flag) continue;
      fence_acquire_agent();
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < kNW; ++j) {
          f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
          for (int s = 0; s < S; ++s) {
            f32x4_t v = (s == ks) ? acc[f][j]
                                  : __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(
                                        part + (int64_t)s * (BM * kBN) +
                                        (((wave * NF + f) * kNW + j) * kWave + lane) * 4));
            sum = (s == 0) ? v : sum + v;
          }
          acc[f][j] = sum;
        }
      if (tid == 0) p.counters[tile] = 0u;
    }

    // ---- epilogue: y = g * acc ----------------------------------------------
    const float gv = p.g[e];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < kNW; ++j) {
        const int col = nrow[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row0 + f * 16 + 4 * q + r;
          if (row < row_end && col < N) {
            const float v = gv * acc[f][j][r];
            if (p.out_f32)
              reinterpret_cast<float*>(p.y)[(int64_t)row * N + col] = v;
            else
              reinterpret_cast<uint16_t*>(p.y)[(int64_t)row * N + col] =
                  (uint16_t)float_to_bf16_rne(v);
          }
        }
      }
  }
}

__global__ void fill_zero_kernel(u32x4_t* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<u32x4_t*>(ptr), n16);
  return hipGetLastError();
}

template <int BM, bool FAST>
static int occupancy() {
  static int occ = -1;
  if (occ < 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemm_kernel<BM, FAST>, kGemmThreads,
                                                     0) != hipSuccess ||
        v < 1)
      v = 1;
    occ = v;
  }
  return occ;
}

static int occupancy_for(int bm, bool fast) {
  switch (bm) {
    case 16: return fast ? occupancy<16, true>() : occupancy<16, false>();
    case 32: return fast ? occupancy<32, true>() : occupancy<32, false>();
    default: return fast ? occupancy<64, true>() : occupancy<64, false>();
  }
}

static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

GemmPlan plan_gemm(int64_t rows, int64_t num_experts, int64_t n, int64_t k, bool grouped,
                   int cu_count) {
  GemmPlan pl{};
  pl.fast = (k % 64) == 0;
  const int64_t avg = grouped ? (rows + num_experts - 1) / (num_experts > 0 ? num_experts : 1)
                              : rows;
  int bm = avg <= 16 ? 16 : (avg <= 32 ? 32 : 64);
  if (grouped && avg > 8 && avg <= 24) bm = 32;  // one row tile for most experts
  const int force_bm = env_int("NVFP4_BM", 0);
  if (force_bm == 16 || force_bm == 32 || force_bm == 64) bm = force_bm;
  pl.bm = bm;
  pl.n_tiles = (int)((n + kBN - 1) / kBN);
  // Upper bound on output tiles: each non-empty expert adds at most one
  // partial row tile beyond rows / bm.
  const int64_t mt_bound = grouped ? (rows + bm - 1) / bm + std::min<int64_t>(num_experts, rows)
                                   : (rows + bm - 1) / bm;
  const int64_t max_tiles = mt_bound * pl.n_tiles;
  const int64_t occ = occupancy_for(bm, pl.fast);
  const int64_t slots = (int64_t)cu_count * occ;
  // Split K only when there are too few tiles to occupy the resident slots.
  const int align = pl.fast ? 64 : 16;
  int splits = 1;
  const int64_t tiles_est = grouped ? std::min<int64_t>(num_experts, rows) * pl.n_tiles
                                    : max_tiles;
  if (tiles_est < slots) {
    int64_t want = (slots + tiles_est - 1) / tiles_est;
    const int64_t kmax = std::max<int64_t>(1, k / kKC);
    splits = (int)std::min<int64_t>(want, kmax);
  }
  const int force_s = env_int("NVFP4_SPLITK", 0);
  if (force_s > 0) splits = force_s;
  if (max_tiles > kMaxCounters) splits = 1;
  int64_t ksplit = (k + splits - 1) / splits;
  ksplit = (ksplit + align - 1) / align * align;
  splits = (int)((k + ksplit - 1) / ksplit);
  pl.splits = splits;
  pl.k_split = (int)ksplit;
  pl.max_tiles = (int)max_tiles;
  const int64_t units_bound = max_tiles * splits;
  pl.grid = (int)std::max<int64_t>(1, std::min<int64_t>(slots, units_bound));
  pl.ws_bytes = splits > 1 ? kCounterBytes + (size_t)max_tiles * splits * bm * kBN * sizeof(float)
                           : 0;
  return pl;
}

hipError_t launch_gemm(const GemmPlan& pl, const GemmParams& p, hipStream_t stream) {
  dim3 grid(pl.grid), block(kGemmThreads);
#define NVFP4_LAUNCH(BMV, FV) \
  hipLaunchKernelGGL((gemm_kernel<BMV, FV>), grid, block, 0, stream, p)
  if (pl.fast) {
    if (pl.bm == 16) NVFP4_LAUNCH(16, true);
    else if (pl.bm == 32) NVFP4_LAUNCH(32, true);
    else NVFP4_LAUNCH(64, true);
  } else {
    if (pl.bm == 16) NVFP4_LAUNCH(16, false);
    else if (pl.bm == 32) NVFP4_LAUNCH(32, false);
    else NVFP4_LAUNCH(64, false);
  }
#undef NVFP4_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
