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
// of the first page.  Unpacked weights are never staged in shared memory
// (staging them was what overflowed it on the pages' hardware, section "The
// Problem Shared Memory Brick Wall" of the same page); only the packed
// 4.5-bit data passes through LDS.
//
// gfx950 design
//  - One persistent grid.  A work unit is (expert, row tile of BM rows,
//    column tile of BN weight rows, K split).  Every workgroup reads the
//    expert offsets from device memory, builds the per-expert unit prefix in
//    LDS and walks units in XCD-aware rounds.  Empty experts own no units.
//    There is no host synchronization.  Workgroups wait for each other only
//    in the fused MoE MLP launch (a down-projection unit waits, with a
//    bounded poll, for the gate_up tiles of its rows) and in the split-K
//    hand-off (the last split to arrive finishes the tile; nobody waits).
//  - MFMA v_mfma_f32_16x16x32_bf16.  Operand A = activations (16 rows),
//    operand B = dequantized weights (16 weight rows = 16 output columns).
//    Lane l holds row/column l % 16 and 8 consecutive K of lane group
//    q = l / 16; which real K a slot carries is a free choice as long as A and
//    B agree, and it is chosen so that each lane's weight bytes are
//    contiguous and its 16 K share one block scale.
//  - Dequant: a nibble pair becomes two exact FP32 values with the gfx950 FP4
//    conversion (scale 1.0; the instruction would apply only the exponent of
//    a scale), is multiplied by the decoded E4M3 block scale (exact), and the
//    upper halves form two BF16 values.  The global scale g is applied once
//    to the FP32 accumulator in the epilogue.
//  - K-phase kernel (k % 64 == 0): weights, activations and scales stream
//    through an LDS ring filled by buffer_load ... lds; each wave owns a
//    column slice and one K half of every stage; row fragments that hold
//    only padding rows of a tile are skipped (the K loop is instantiated per
//    number of occupied fragments).  Details at the kernel.
//  - Large-M kernel (dense, k % 64 == 0, hundreds of rows): 256 x 256 tiles,
//    v_mfma_f32_32x32x16_bf16, each wave on all 256 rows of 32 columns.
//    Details at the kernel.
//  - Register kernel (any k % 16 == 0): 4 waves x 64 columns, weights loaded
//    straight into registers one 256-wide chunk ahead, activations staged
//    through a double-buffered LDS tile.
//  - Split-K (used when there are too few output tiles to fill the chip):
//    each split writes its FP32 partial tile to the workspace, bumps the
//    tile's counter, and the last arrival sums the partials in split order
//    (bitwise reproducible), resets the counter and writes the output.
#include <algorithm>
#include <type_traits>
#include <atomic>
#include <mutex>
#include <cstdlib>

#include "device_common.hpp"
#include "kp_layout.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

// ---- shared pieces ----------------------------------------------------------

// Buffer resource over [base, base + bytes) for raw (stride 0) buffer loads:
// offsets at or beyond `bytes` read as zero, which masks rows past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr uint32_t kOffNone = 0x80000000u;  // beyond every resource: loads return 0

// Cache policy of buffer accesses that must be coherent across the XCDs'
// L2 caches (device scope): the sc1 bit.  Such stores write through to
// memory and such loads do not hit lines another XCD may have left stale.
constexpr int kCpolDevice = 16;

// Exclusive scan of one int per thread over a workgroup of THREADS threads.
template <int THREADS>
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
  for (int w = 0; w < THREADS / kWave; ++w) {
    base += (w < wave) ? tmp[w] : 0;
    sum += tmp[w];
  }
  __syncthreads();
  *total = sum;
  return base + incl - v;
}

// Per-workgroup schedule in dynamic LDS (sized at launch).  Units are
// enumerated expert by expert in a schedule order; for each position of that
// order the LDS holds the exclusive prefix of work units.
//  - Up to kSortMax experts: the experts are taken in order of decreasing row
//    count (ties by id), so the rounds of a persistent launch start with the
//    costliest units and end with the cheapest ones, and the last, partly
//    filled round holds short units; the LDS also caches each expert's
//    segment start and global scale, so a unit is decoded without a memory
//    round trip.  Layout: units [E + 1], expert of each position [E],
//    segment starts [E + 1], global scales [E].
//  - More experts: id order, units [E + 1] only; segment bounds and global
//    scales come through the scalar cache.
extern __shared__ int sched_units[];
constexpr int kSortMax = 256;
constexpr int kSchedLdsMax = 4 * (4 * kSortMax + 2) > 4 * (kMaxExperts + 1)
                                 ? 4 * (4 * kSortMax + 2)
                                 : 4 * (kMaxExperts + 1);
inline int sched_lds_bytes(int64_t num_experts) {
  return num_experts <= kSortMax ? (int)(4 * (4 * num_experts + 2)) : (int)(4 * (num_experts + 1));
}
__device__ __forceinline__ int* sched_perm(int E) { return sched_units + E + 1; }
__device__ __forceinline__ int* sched_seg(int E) { return sched_units + 2 * E + 1; }
__device__ __forceinline__ float* sched_g(int E) {
  return reinterpret_cast<float*>(sched_units + 3 * E + 2);
}
struct Sched {
  int tmp[16];
  int flag;
};

// A uniform 32-bit load through the scalar cache (the data are inputs this
// kernel never writes, so the load needs no ordering against its stores);
// it waits on the LDS/scalar counter only, so loads in flight on the vector
// memory counter are not waited for.
__device__ __forceinline__ uint32_t sload_u32(const void* base, uint32_t byte_off) {
  // the address is uniform; say so, so that it stays in SGPRs
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t ua = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32);
  uint32_t v;
  asm volatile("s_load_dword %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(v)
               : "s"(ua), "s"(__builtin_amdgcn_readfirstlane(byte_off)));
  return v;
}

// Four dwords at byte_off of a buffer through the scalar cache (bounds-
// checked: bytes past the resource read as zero).  A scalar load counts in
// lgkmcnt, not in the vector-memory counter the K-phase waits rely on.
__device__ __forceinline__ u32x4_t sbuffer_load_x4(u32x4_t rsrc, uint32_t byte_off) {
  rsrc = u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane(rsrc[0]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[1]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[2]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[3])};
  u32x4_t v;
  asm volatile("s_buffer_load_dwordx4 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(v)
               : "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(byte_off)));
  return v;
}

__device__ __forceinline__ int seg_begin(const GemmParams& p, int e) {
  return p.offsets ? p.offsets[e] : (e == 0 ? 0 : (int)p.rows);
}

// Fills `sc` and the LDS schedule; returns the total unit count, or -1
// (after flagging the status word) when the offsets are malformed.
template <int THREADS, int BM>
__device__ __forceinline__ int build_schedule(Sched& sc, const GemmParams& p) {
  const int tid = threadIdx.x;
  const int E = p.num_experts;
  const bool sorted = E <= kSortMax;
  constexpr int PER = (kMaxExperts + THREADS - 1) / THREADS;  // experts per thread
  int bad = 0;
  int cnt[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = PER * tid + t;
    cnt[t] = 0;
    if (e < E) {
      const int a = seg_begin(p, e), b = seg_begin(p, e + 1);
      bad |= b < a;
      cnt[t] = (b - a + BM - 1) / BM * p.n_tiles * p.splits;
      if (sorted) {
        sched_seg(E)[e] = a;
        sched_g(E)[e] = p.g[e];
      }
    }
  }
  if (tid == 0) {
    bad |= (seg_begin(p, 0) != 0) || ((int64_t)seg_begin(p, E) != p.rows);
    if (sorted) sched_seg(E)[E] = seg_begin(p, E);
  }
  bad = __syncthreads_or(bad);
  if (bad) {
    if (blockIdx.x == 0 && tid == 0 && p.d_status != nullptr)
      atomicOr(p.d_status, NVFP4_DSTATUS_BAD_OFFSETS);
    return -1;
  }
  if (sorted) {
    // position of expert e: experts with more rows, then equal rows and a
    // smaller id, come first (the same order in every workgroup); its unit
    // count goes to that position
    static_assert(THREADS >= kSortMax, "one expert per thread when sorting");
    const int* seg = sched_seg(E);
    if (tid < E) {
      const int r = seg[tid + 1] - seg[tid];
      int pos = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const int r2 = seg[e2 + 1] - seg[e2];
        pos += (r2 > r) || (r2 == r && e2 < tid);
      }
      sched_perm(E)[pos] = tid;
      sched_units[pos] = (r + BM - 1) / BM * p.n_tiles * p.splits;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int pos = PER * tid + t;
      cnt[t] = pos < E ? sched_units[pos] : 0;
    }
    __syncthreads();
  }
  int my_units = 0;
#pragma unroll
  for (int t = 0; t < PER; ++t) my_units += cnt[t];
  int total_units;
  int ubase = block_exclusive_scan<THREADS>(my_units, sc.tmp, &total_units);
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int pos = PER * tid + t;
    if (pos < E) sched_units[pos] = ubase;
    ubase += cnt[t];
  }
  if (tid == 0) sched_units[E] = total_units;
  __syncthreads();
  return total_units;
}

// Global scale of expert e.
__device__ __forceinline__ float expert_g(const GemmParams& p, int e) {
  return p.num_experts <= kSortMax ? sched_g(p.num_experts)[e]
                                   : __uint_as_float(sload_u32(p.g, 4u * (uint32_t)e));
}

struct Unit {
  int e, ks, nt, tile, row0, row_end, k_beg, k_end;
  int rt;  // row tile of the launch (experts' row tiles in schedule order)
};

// Work units are handed out in rounds of gridDim.x.  Within a round, unit
// ids are placed XCD-major: the hardware dispatches workgroup w to XCD
// w % 8, so consecutive unit ids -- the row tiles of one expert's weight
// tile, then its other column tiles -- go to workgroups w, w+8, w+16, ... of
// one XCD and stream the same weight bytes through that XCD's L2 at about
// the same time instead of each fetching them from HBM.  The map is a
// bijection of [0, G) onto itself, so every unit is processed exactly once.
__device__ __forceinline__ int round_unit(int round, int w, int G) {
  const int in_round = (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
  return round * G + in_round;
}

// The K-phase kernel's units are sorted by cost (the experts with the most
// rows first), so a plain round-robin hands workgroup 0 the costliest unit
// of every round and the last workgroup the cheapest.  Odd rounds therefore
// take the round's ids in reverse order (each XCD's block of ids stays
// contiguous), which evens out the workgroups' totals (1-2 % on the MoE
// launches; what remains idle at their end is the last, partly filled
// round, not the cost order).
__device__ __forceinline__ int snake_unit(int round, int w, int G) {
  const int in_round = (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
  return round * G + ((round & 1) ? G - 1 - in_round : in_round);
}

// Units of expert e are ordered (column tile, split, row tile); the expert's
// output tiles (for the split-K counters) are numbered units / splits.
// P2: the second product of a fused launch, whose units (p.n_tiles column
// tiles per row tile, no K split) follow the schedule built for the first
// product's n1 column tiles: its unit prefix is the first's scaled by
// p.n_tiles / n1.
template <int BM, bool P2 = false>
__device__ __forceinline__ Unit decode_unit(const Sched& sc, const GemmParams& p, int unit,
                                            int n1 = 1) {
  auto prefix = [&](int pos) {
    return P2 ? sched_units[pos] / n1 * p.n_tiles : sched_units[pos];
  };
  // schedule position: last one with units[pos] <= unit (empty experts have
  // equal bounds)
  const int E = p.num_experts;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix(mid) <= unit) lo = mid; else hi = mid;
  }
  const int pos = __builtin_amdgcn_readfirstlane(lo);
  Unit u;
  int seg0, seg1;
  if (E <= kSortMax) {
    u.e = __builtin_amdgcn_readfirstlane(sched_perm(E)[pos]);
    seg0 = __builtin_amdgcn_readfirstlane(sched_seg(E)[u.e]);
    seg1 = __builtin_amdgcn_readfirstlane(sched_seg(E)[u.e + 1]);
  } else {
    u.e = pos;
    // segment bounds through the scalar cache: a vector load here would make
    // the compiler wait for every load in flight, prefetched stages included
    seg0 = p.offsets ? (int)sload_u32(p.offsets, 4u * (uint32_t)u.e) : 0;
    seg1 = p.offsets ? (int)sload_u32(p.offsets, 4u * (uint32_t)(u.e + 1)) : (int)p.rows;
  }
  const int mtiles = (seg1 - seg0 + BM - 1) / BM;
  const int local = unit - prefix(pos);
  const int mt = local % mtiles;
  const int rest = local / mtiles;
  u.ks = rest % p.splits;
  u.nt = rest / p.splits;
  u.tile = prefix(pos) / p.splits + u.nt * mtiles + mt;
  u.rt = (P2 ? sched_units[pos] / n1 : sched_units[pos] / (p.n_tiles * p.splits)) + mt;
  u.row0 = seg0 + mt * BM;
  u.row_end = min(u.row0 + BM, seg1);
  u.k_beg = u.ks * p.k_split;
  u.k_end = min(p.k, u.k_beg + p.k_split);
  return u;
}

// Split-K hand-off and epilogue for a workgroup of WAVES waves over a BN-wide
// column tile, each wave holding NF x NW MFMA accumulator tiles
// (column = nt*BN + wave*NW*16 + j*16 + l%16, row = row0 + f*16 + 4*(l/16) + r).
// Returns false when another split of the tile will finish it.
template <int NF, int NW, int WAVES, int BN>
__device__ __forceinline__ bool finish_tile(f32x4_t (&acc)[NF][NW], const GemmParams& p,
                                            const Unit& u, float gv, Sched& sc) {
  constexpr int BM = NF * 16;
  static_assert(WAVES * NW * 16 == BN, "waves cover the column tile");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = p.splits;
  if (S > 1) {
    // Hand-off between the splits of a tile, which may run on different XCDs
    // (each with its own L2).  The partials are written and read with
    // device-scope accesses, which go past the non-coherent L2, and each
    // thread waits for its stores to complete before the barrier that
    // precedes the arrival count; so no whole-L2 writeback or invalidate
    // (what a device-scope fence costs) is needed.
    const __amdgpu_buffer_rsrc_t part =
        make_rsrc(p.partials + (int64_t)u.tile * S * (BM * BN), (uint32_t)(S * BM * BN * 4));
    // byte offset of this lane's accumulator tile (f, j) in split s
    auto poff = [&](int s, int f, int j) {
      return (uint32_t)((s * (BM * BN) + (((wave * NF + f) * NW + j) * kWave + lane) * 4) * 4);
    };
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < NW; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[f][j]), part,
                                               poff(u.ks, f, j), 0, kCpolDevice);
    __builtin_amdgcn_s_waitcnt(0);  // every counter at zero: the stores have completed
    __syncthreads();
    if (tid == 0) {
      const uint32_t old =
          __hip_atomic_fetch_add(&p.counters[u.tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sc.flag = (old == (uint32_t)(S - 1));
    }
    __syncthreads();
    if (!sc.flag) return false;
    // Sum the partials in split order.  U splits are loaded before any is
    // added, so about 8 independent loads are in flight instead of one.
    constexpr int U = NF * NW >= 8 ? 1 : 8 / (NF * NW);
    f32x4_t sum[NF][NW];
    for (int s0 = 0; s0 < S; s0 += U) {
      f32x4_t v[U][NF][NW];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int s = s0 + i;
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int j = 0; j < NW; ++j)
            v[i][f][j] = (s >= S || s == u.ks)
                             ? acc[f][j]
                             : __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                               part, poff(s, f, j), 0, kCpolDevice));
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (s0 + i >= S) break;
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int j = 0; j < NW; ++j)
            sum[f][j] = (s0 + i == 0) ? v[i][f][j] : sum[f][j] + v[i][f][j];
      }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < NW; ++j) acc[f][j] = sum[f][j];
    if (tid == 0) __hip_atomic_store(&p.counters[u.tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int q = lane >> 4, r16 = lane & 15;
  // Output value and column of accumulator element (f, j, r) at column col,
  // or false when it writes nothing.  With the SiLU(gate) * up epilogue the
  // weight rows come in 32-row groups (16 gate rows, then the 16 up rows of
  // the same outputs), so the wave's even column tile j holds gate values
  // and tile j + 1 the matching up values; odd tiles write nothing.
  const bool glu = p.act != 0;
  const int nout = glu ? p.n / 2 : p.n;
  auto element = [&](int f, int j, int r, int col, int row, float& v, int& ocol) {
    if (!(row < u.row_end && col < p.n)) return false;
    if (!glu) {
      v = gv * acc[f][j][r];
      ocol = col;
      return true;
    }
    if ((j & 1) || NW % 2) return false;
    const float gate = gv * acc[f][j][r];
    const float up = gv * acc[f][(j + 1) % NW][r];
    // SiLU(gate) = gate / (1 + e^-gate), with e^-gate = 2^(-gate log2 e) on
    // the hardware exp2 and the hardware reciprocal: relative error ~1e-6,
    // far inside the FP32 output's bound (1e-5 of the error scale)
    const float e = __builtin_amdgcn_exp2f(-gate * 1.4426950408889634f);
    v = gate * __builtin_amdgcn_rcpf(1.0f + e) * up;
    ocol = (col - r16) / 2 + r16;  // col - r16 is a multiple of 32
    return true;
  };
  if (p.n <= kFixedStoreMaxN) {
    // One buffer store per accumulator element, always issued (elements
    // that write nothing get an offset past the resource and are dropped),
    // so this epilogue issues exactly 4 NF NW vector memory instructions.
    const int esz = p.out_f32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(static_cast<const char*>(p.y) + (int64_t)u.row0 * nout * esz,
                  (uint32_t)((u.row_end - u.row0) * nout * esz));
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const int col = u.nt * BN + wave * (NW * 16) + j * 16 + r16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = u.row0 + f * 16 + 4 * q + r;
          float v = 0.f;
          int ocol = 0;
          const uint32_t off = element(f, j, r, col, row, v, ocol)
                                   ? (uint32_t)(((row - u.row0) * nout + ocol) * esz)
                                   : kOffNone;
          if (p.out_f32)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)float_to_bf16_rne(v), ry, off, 0, 0);
        }
      }
    return true;
  }
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int col = u.nt * BN + wave * (NW * 16) + j * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = u.row0 + f * 16 + 4 * q + r;
        float v = 0.f;
        int ocol = 0;
        if (element(f, j, r, col, row, v, ocol)) {
          if (p.out_f32)
            reinterpret_cast<float*>(p.y)[(int64_t)row * nout + ocol] = v;
          else
            reinterpret_cast<uint16_t*>(p.y)[(int64_t)row * nout + ocol] =
                (uint16_t)float_to_bf16_rne(v);
        }
      }
    }
  return true;
}

// ---- staged-ring pieces (k % 64 == 0) ---------------------------------------------


// ---- K-phase kernel (k % 64 == 0) ----------------------------------------------
//
// A work unit is (expert, row tile of BM rows, column tile of BN = 128 or 256
// weight rows, K split).  K advances in 128-wide stages held in an
// NSLOT-deep LDS ring: packed weights (BN rows x 64 B), the activation tile
// (BM rows x 256 B), and block scales in windows of 4 stages (BN rows x
// 32 B), all written by buffer_load ... lds (no register staging).
//
// The KW waves split the work as wave w = 2 ch + kp: it owns the
// CPW = 2 BN / KW columns [CPW ch, CPW ch + CPW) and the K half
// [64 kp, 64 kp + 64) of every stage.  Each wave thus reads only half of the
// staged activation tile, and its column tiles share every activation
// fragment; the two K halves of a column are summed through LDS once per
// unit.  Operands of stage c + 1 are read from LDS into registers while stage
// c is multiplied out, so LDS latency hides behind a whole stage of
// dequantization and MFMA; NSLOT - 2 stages are in flight from HBM meanwhile.
//
// Small tiles run as 4-wave workgroups on 128 columns, two workgroups per
// CU: the two waves that share a SIMD then belong to different workgroups,
// so the SIMD's issue arbitration (which favours the older wave) never makes
// one of them wait for the other at a barrier.
//
// LDS swizzles (chosen for gfx950's ds_read_b128 / ds_read_b64 bank mapping):
// activation row r keeps its 16-byte chunk c in slot c ^ (r & 15); weight row
// R keeps its 16-byte chunk c in slot c ^ ((R >> 2) & 3).
// LDS budget of every K-phase configuration: ring, scale windows, the
// workgroup's schedule scratch and the largest dynamic schedule.
template <int BM, int NSLOT, int KW, int BN>
constexpr bool kp_fits_lds() {
  return KpLayout<BM, NSLOT, KW, BN>::kTotal + (int)sizeof(Sched) + kSchedLdsMax <= 160 * 1024;
}

template <int BM, int KW, int BN>
struct KpOffsets {
  uint32_t w[KpLayout<BM, 4, KW, BN>::kWPerWave];
  uint32_t x[KpLayout<BM, 4, KW, BN>::kXPerWave];
  int xk[KpLayout<BM, 4, KW, BN>::kXPerWave];
  uint32_t s[2];
};

// Per-lane offsets of a wave's loads, relative to the unit's first weight
// row and first activation row (the same for every unit).
template <int BM, int NSLOT, int KW, int BN>
__device__ __forceinline__ KpOffsets<BM, KW, BN> kp_offsets(int K, int wave, int lane) {
  using L = KpLayout<BM, NSLOT, KW, BN>;
  KpOffsets<BM, KW, BN> o;
  // weights: load t covers rows 16t..16t+15 (64 B each); slot s of row R
  // receives chunk s ^ ((R >> 2) & 3)
#pragma unroll
  for (int tt = 0; tt < L::kWPerWave; ++tt) {
    const int R = (wave * L::kWPerWave + tt) * 16 + (lane >> 2);
    const int g = (lane & 3) ^ ((R >> 2) & 3);
    o.w[tt] = (uint32_t)R * (uint32_t)(K / 2) + (uint32_t)(16 * g);
  }
  // activations: load t covers rows 4t..4t+3 (256 B each); slot s of row r
  // receives chunk s ^ (r & 15).  With fewer loads than waves, waves repeat
  // a load (same bytes to the same place) so every wave issues the same count.
#pragma unroll
  for (int tt = 0; tt < L::kXPerWave; ++tt) {
    const int t = L::kXInstr >= KW ? wave * L::kXPerWave + tt : wave % L::kXInstr;
    const int r = t * 4 + (lane >> 4);
    const int g = (lane & 15) ^ (r & 15);
    o.x[tt] = (uint32_t)r * (uint32_t)(K * 2) + (uint32_t)(16 * g);
    o.xk[tt] = 8 * g;
  }
  // scale window: 1 KB loads of 1024 / kWinRow rows, kSPerWave per wave
  // (waves beyond the load count repeat a load)
  static_assert(L::kSPerWave <= 2, "scale loads per wave");
#pragma unroll
  for (int tt = 0; tt < L::kSPerWave; ++tt) {
    constexpr int LPR = L::kWinRow / 16;  // lanes per row
    const int t = L::kSInstr >= KW ? wave * L::kSPerWave + tt : wave % L::kSInstr;
    const int R = t * (64 / LPR) + lane / LPR;
    o.s[tt] = (uint32_t)R * (uint32_t)(K / 16) + (uint32_t)(16 * (lane % LPR));
  }
  return o;
}

// A unit's load sources: buffer descriptors based at its expert's first
// weight row of the column tile and at its first activation row, and its K
// range in 128-deep stages.
struct KpU {
  u32x4_t rw, rs, rx;
  int k_beg, k_end, nch;
};

template <int BN>
__device__ __forceinline__ KpU kp_unit(const GemmParams& p, const Unit& u) {
  const int N = p.n, K = p.k;
  const int n0 = u.nt * BN;
  KpU s;
  s.rw = rsrc_words(p.w + ((int64_t)u.e * N + n0) * (K / 2), (uint32_t)(N - n0) * (uint32_t)(K / 2));
  s.rs = rsrc_words(p.s + ((int64_t)u.e * N + n0) * (K / 16), (uint32_t)(N - n0) * (uint32_t)(K / 16));
  s.rx = rsrc_words(p.x + (int64_t)u.row0 * K, (uint32_t)(u.row_end - u.row0) * (uint32_t)(K * 2));
  s.k_beg = u.k_beg;
  s.k_end = u.k_end;
  s.nch = (u.k_end - u.k_beg + kRingKC - 1) / kRingKC;
  return s;
}

// TAIL: the stage may reach past the end of the unit's K range (only its
// last stage can).
// G: the unit's activation rows come through a row index (per-unit offsets
// in u.xg instead of the unit-independent o.x).
// COH: the activations come from the first product of a fused launch
// (device-coherent loads).
template <int BM, int NSLOT, int KW, int BN, bool TAIL = true, bool G = false, bool COH = false>
__device__ __forceinline__ void kp_issue(uint32_t stage, u32x4_t rw, u32x4_t rx,
                                         const KpOffsets<BM, KW, BN>& o, int kc, int k_end,
                                         int wave, uint32_t xg0 = 0, uint32_t xg1 = 0) {
  using L = KpLayout<BM, NSLOT, KW, BN>;
#pragma unroll
  for (int tt = 0; tt < L::kWPerWave; ++tt)
    lds_dma16(stage + L::kW + (wave * L::kWPerWave + tt) * 1024, o.w[tt], (uint32_t)(kc / 2), rw);
  const bool tail = TAIL && kc + kRingKC > k_end;
#pragma unroll
  for (int tt = 0; tt < L::kXPerWave; ++tt) {
    const int t = L::kXInstr >= KW ? wave * L::kXPerWave + tt : wave % L::kXInstr;
    const uint32_t xo = G ? (tt == 0 ? xg0 : xg1) : o.x[tt];
    const uint32_t voff = (tail && kc + o.xk[tt] >= k_end) ? kOffNone : xo;
    lds_dma16<COH>(stage + L::kX + t * 1024, voff, (uint32_t)(kc * 2), rx);
  }
}

// Activation sources of a unit whose rows come through p.row_index: the
// buffer spans the whole token matrix, and each lane's load offset follows
// its row's index.  Load t of a wave covers tile rows 4t .. 4t+3 (lane group
// lane / 16), so one scalar load brings the four indices of each load.  Rows
// past the tile, and indices outside [0, x_rows), load nothing (zeros); the
// latter set NVFP4_DSTATUS_BAD_INDEX.
template <int BM, int NSLOT, int KW, int BN>
__device__ __forceinline__ void kp_gather(KpU& s, uint32_t (&xg)[2], const GemmParams& p,
                                          const Unit& u, int wave, int lane) {
  using L = KpLayout<BM, NSLOT, KW, BN>;
  static_assert(L::kXPerWave <= 2, "gather offsets per wave");
  const uint32_t row_bytes = (uint32_t)p.k * 2u;
  s.rx = rsrc_words(p.x, (uint32_t)p.x_rows * row_bytes);
  const u32x4_t ri = rsrc_words(p.row_index + u.row0, (uint32_t)(u.row_end - u.row0) * 4u);
  const int q = lane >> 4;
  bool bad = false;
#pragma unroll
  for (int tt = 0; tt < L::kXPerWave; ++tt) {
    const int t = L::kXInstr >= KW ? wave * L::kXPerWave + tt : wave % L::kXInstr;
    if (4 * t >= u.row_end - u.row0) {  // the load's four rows are all past the tile
      xg[tt] = kOffNone;
      continue;
    }
    const u32x4_t idx = sbuffer_load_x4(ri, (uint32_t)(16 * t));
    const uint32_t tok = q == 0 ? idx[0] : (q == 1 ? idx[1] : (q == 2 ? idx[2] : idx[3]));
    const int r = 4 * t + q;
    const int g = (lane & 15) ^ (r & 15);
    const bool row_ok = u.row0 + r < u.row_end;
    const bool tok_ok = tok < (uint32_t)p.x_rows;  // also rejects negative indices
    bad |= row_ok && !tok_ok;
    xg[tt] = (row_ok && tok_ok) ? tok * row_bytes + (uint32_t)(16 * g) : kOffNone;
  }
  if (bad && p.d_status != nullptr) atomicOr(p.d_status, NVFP4_DSTATUS_BAD_INDEX);
}

// Issue the scale window [kw, kw + 128 kWinStages) of the unit (one 1 KB load
// per wave).
template <int BM, int NSLOT, int KW, int BN>
__device__ __forceinline__ void kp_issue_scales(uint32_t slot, u32x4_t rs,
                                                const KpOffsets<BM, KW, BN>& o, int kw, int wave) {
  using L = KpLayout<BM, NSLOT, KW, BN>;
#pragma unroll
  for (int tt = 0; tt < L::kSPerWave; ++tt) {
    const int t = L::kSInstr >= KW ? wave * L::kSPerWave + tt : wave % L::kSInstr;
    lds_dma16(slot + t * 1024, o.s[tt], (uint32_t)(kw / 16), rs);
  }
}

// One stage's operands of one wave: per column tile j, 16 nibbles (two MFMA
// K steps) and one E4M3 block scale; per K step i and row tile f, one
// activation fragment.
template <int BM, int NJ>
struct KpRegs {
  u32x2_t wd[NJ];
  uint32_t sc[NJ];
  bool kv;  // the lane's scale block lies inside the unit's K range
  bf16x8_t a[2][BM / 16];
};

// Lane group q of wave half kp supplies K = 64 kp + 16 q + 8 i .. +7 of the
// stage in MFMA step i: its 16 K are one scale block (block 4 kp + q of the
// stage), 8 contiguous weight bytes and two 16-byte activation chunks.
template <int BM, int NJ, int NFE, int BN, int WS>
__device__ __forceinline__ void kp_read(KpRegs<BM, NJ>& r, const uint8_t* stage,
                                        const uint8_t* swin, int sub, bool kvalid, int kp,
                                        int ch, int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  const int cw = 2 * kp + (q >> 1);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int R = ch * (NJ * 16) + j * 16 + r16;
    r.wd[j] = *reinterpret_cast<const u32x2_t*>(stage + R * 64 + 16 * (cw ^ ((R >> 2) & 3)) +
                                                8 * (q & 1));
    r.sc[j] = swin[R * (8 * WS) + 8 * sub + 4 * kp + q];
  }
  r.kv = kvalid;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < NFE; ++f)
      r.a[i][f] = *reinterpret_cast<const bf16x8_t*>(stage + BN * 64 + (f * 16 + r16) * 256 +
                                                     16 * ((8 * kp + 2 * q + i) ^ r16));
}

// Multiply out one stage held in registers.  The B fragment of step t + 1
// is dequantized while the MFMAs of step t run.
template <int BM, int NJ, int NFE>
__device__ __forceinline__ void kp_mma(f32x4_t (&acc)[BM / 16][NJ], const KpRegs<BM, NJ>& r) {
  float scl[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) scl[j] = r.kv ? decode_e4m3<0>(r.sc[j]) : 0.f;
  constexpr int T = 2 * NJ;
  bf16x8_t b[2];
  b[0] = dequant8(r.wd[0][0], scl[0]);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int i = t / NJ, j = t % NJ;
    if (t + 1 < T) {
      const int i1 = (t + 1) / NJ, j1 = (t + 1) % NJ;
      b[(t + 1) & 1] = dequant8(r.wd[j1][i1], scl[j1]);
    }
#pragma unroll
    for (int f = 0; f < NFE; ++f)
      acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.a[i][f], b[t & 1], acc[f][j], 0, 0, 0);
  }
}

// Dependency of a unit of a fused launch's second product: the count of
// stored first-product column tiles of its row tile must reach `target`.
// Each wave polls on its own (the count only grows, so the waves of a
// workgroup agree).  A wave gives up after `limit` polls, sets
// NVFP4_DSTATUS_WAIT_TIMEOUT and from then on does not wait at all
// (`gave_up`), so a launch whose workgroups are not all resident still ends.
struct KpWait {
  const uint32_t* ctr;  // nullptr: nothing to wait for
  uint32_t target;
  int limit;
  uint32_t* d_status;
};

__device__ __forceinline__ void kp_wait(const KpWait& w, bool& gave_up) {
  if (w.ctr == nullptr || gave_up) return;
  for (int i = 0;; ++i) {
    const uint32_t v = __hip_atomic_load(w.ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= w.target) return;
    if (i >= w.limit) {
      gave_up = true;
      if (w.d_status != nullptr) atomicOr(w.d_status, NVFP4_DSTATUS_WAIT_TIMEOUT);
      return;
    }
    __builtin_amdgcn_s_sleep(4);
  }
}

// The K loop of one unit, for tiles whose rows fill NFE of the BM / 16 row
// fragments (fragments past NFE are pure padding and are skipped).
//
// The workgroup's units form one stream of stages: stage c of a unit lives
// in ring slot (sb0 + c) % NSLOT and window i of a unit in buffer
// (wb0 + i) % 3.  Per unit (per wave, in issue order): stages 0 .. NSLOT-1,
// each preceded by the scale window that starts at it (every WS-th stage).
// The first `pf` of them may already be in flight, issued during the
// previous unit's last iterations and followed there by `ex` epilogue
// stores.  Iteration c waits until stage c + 1 has landed and passes the
// barrier: every wave has then read stage c into registers (in iteration
// c - 1, or before the loop when c = 0), so stage c's slot takes stage
// c + NSLOT -- or, in the unit's last iterations, one of the next unit's
// first `pn` stages.  It then reads stage c + 1 into registers and
// multiplies out stage c.
//
// While the stage issued lies inside the unit's K range (the last stage only
// when it is full), the iterations run in blocks of WS whose waits, window
// issues and K checks are compile-time constants; the remaining iterations
// take the general path.
// COH: device-coherent activation loads (second product of a fused launch);
// nxw: what the next unit waits for before its first prefetched load.
template <int BM, int NSLOT, int KW, int BN, int NFE, bool G, bool COH = false>
__device__ __forceinline__ void kp_kloop(f32x4_t (&acc)[BM / 16][2 * BN / KW / 16],
                                         uint8_t* ring, const KpU& cu, int sb0, int wb0, int pf,
                                         bool ex, const KpU& nx, int pn, uint32_t cxg0,
                                         uint32_t cxg1, uint32_t nxg0, uint32_t nxg1,
                                         const KpOffsets<BM, KW, BN>& off, int kp, int ch,
                                         int wave, int lane, const KpWait& nxw, bool& gave_up) {
  using L = KpLayout<BM, NSLOT, KW, BN>;
  constexpr int NJ = L::kNJ;
  constexpr int D = NSLOT;  // stages in flight after an iteration's issue
  constexpr int WS = L::kWinStages;
  constexpr int LS = L::kLoadsPerStage;
  constexpr int SPW = L::kSPerWave;
  constexpr int E = L::kEpiStores;
  static_assert(WS % 2 == 0, "blocks keep the register double buffer in phase");
  const int q = lane >> 4;
  const uint32_t ring0 = lds_addr(ring);
  const int nch = cu.nch;
  const int nwin = (nch + WS - 1) / WS;
  auto slot = [&](int c) { return ((sb0 + c) % NSLOT) * L::kStage; };
  auto wbuf = [&](int i) { return L::kSWin + ((wb0 + i) % L::kWinBufs) * L::kWinBytes; };
  // K validity of this lane's scale block in stage c
  auto kvalid = [&](int c) { return cu.k_beg + c * kRingKC + 64 * kp + 16 * q < cu.k_end; };
  auto issue_stage = [&](int st) {
    if (st % WS == 0)
      kp_issue_scales<BM, NSLOT, KW, BN>(ring0 + wbuf(st / WS), cu.rs, off,
                                         cu.k_beg + st * kRingKC, wave);
    kp_issue<BM, NSLOT, KW, BN, true, G, COH>(ring0 + slot(st), cu.rw, cu.rx, off,
                                              cu.k_beg + st * kRingKC, cu.k_end, wave, cxg0,
                                              cxg1);
  };
  // loads this wave issued after those of stage lo, through stage hi, plus
  // the previous unit's epilogue stores when stage lo was issued before them
  auto loads_after = [&](int lo, int hi) {
    int n = (ex && lo < pf) ? E : 0;
#pragma unroll
    for (int i = 1; i < D; ++i)
      if (lo + i <= hi) n += LS + ((lo + i) % WS == 0 ? SPW : 0);
    return n;
  };
  int nx_ops = 0;  // loads issued for the next unit so far
  for (int st = pf; st < D && st < nch; ++st) issue_stage(st);
  wait_vmcnt(loads_after(0, min(D, nch) - 1));
  __syncthreads();
  KpRegs<BM, NJ> ra, rb;
  kp_read<BM, NJ, NFE, BN, WS>(ra, ring + slot(0), ring + wbuf(0), 0, kvalid(0), kp, ch, lane);

  // iteration c = c0 + T of a steady block (c0 % WS == 0): stages c + 1 ..
  // c + D - 1 are in flight and full, stage c + D is full
  auto steady = [&](auto tc, int c0, const KpRegs<BM, NJ>& cur, KpRegs<BM, NJ>& nxt) {
    constexpr int T = decltype(tc)::value;
    constexpr int kAfter = [] {
      int n = 0;
      for (int i = 2; i < D; ++i) n += LS + ((T + i) % WS == 0 ? SPW : 0);
      return n;
    }();
    const int c = c0 + T;
    if (ex && c + 1 < pf) wait_vmcnt_c<kAfter + E>();
    else wait_vmcnt_c<kAfter>();
    __syncthreads();
    if constexpr ((T + D) % WS == 0)
      kp_issue_scales<BM, NSLOT, KW, BN>(ring0 + wbuf((c + D) / WS), cu.rs, off,
                                         cu.k_beg + (c + D) * kRingKC, wave);
    kp_issue<BM, NSLOT, KW, BN, false, G, COH>(ring0 + slot(c + D), cu.rw, cu.rx, off,
                                               cu.k_beg + (c + D) * kRingKC, cu.k_end, wave,
                                               cxg0, cxg1);
    kp_read<BM, NJ, NFE, BN, WS>(nxt, ring + slot(c + 1), ring + wbuf((c + 1) / WS), (T + 1) % WS,
                                 true, kp, ch, lane);
    kp_mma<BM, NJ, NFE>(acc, cur);
  };
  auto step = [&](int c, const KpRegs<BM, NJ>& cur, KpRegs<BM, NJ>& nxt) {
    if (c + 1 < nch) {
      // stages c + 1 .. min(c + D - 1, nch - 1) are in flight, then the
      // next unit's loads issued so far
      wait_vmcnt(loads_after(c + 1, min(c + D - 1, nch - 1)) + nx_ops);
      __syncthreads();
      if (c + D < nch) {
        issue_stage(c + D);
      } else if (c + D - nch < pn) {
        // the next unit's stage j goes where this unit's stage c was; its
        // first window (j = 0) goes first
        const int j = c + D - nch;
        if (j == 0) {
          kp_wait(nxw, gave_up);  // the next unit's activations are stored
          kp_issue_scales<BM, NSLOT, KW, BN>(ring0 + wbuf(nwin), nx.rs, off, nx.k_beg, wave);
          nx_ops += SPW;
        }
        kp_issue<BM, NSLOT, KW, BN, true, G, COH>(ring0 + slot(c + D), nx.rw, nx.rx, off,
                                                  nx.k_beg + j * kRingKC, nx.k_end, wave, nxg0,
                                                  nxg1);
        nx_ops += LS;
      }
      kp_read<BM, NJ, NFE, BN, WS>(nxt, ring + slot(c + 1), ring + wbuf((c + 1) / WS),
                                   (c + 1) % WS, kvalid(c + 1), kp, ch, lane);
    }
    kp_mma<BM, NJ, NFE>(acc, cur);
  };
  const bool full_last = cu.k_end - cu.k_beg == nch * kRingKC;
  const int c_lim = nch - WS - D + (full_last ? 1 : 0);
  int c = 0;
  for (; c < c_lim; c += WS) {
    steady(std::integral_constant<int, 0>{}, c, ra, rb);
    steady(std::integral_constant<int, 1>{}, c, rb, ra);
    if constexpr (WS == 4) {
      steady(std::integral_constant<int, 2>{}, c, ra, rb);
      steady(std::integral_constant<int, 3>{}, c, rb, ra);
    }
  }
  for (; c < nch; c += 2) {
    step(c, ra, rb);
    if (c + 1 < nch) step(c + 1, rb, ra);
  }
}

// Epilogue of a unit without a K split, through LDS.  Wave w holds the
// summed accumulators of columns [16 NH w, 16 NH (w + 1)) of the unit (NH
// 16-column tiles, NF 16-row fragments).  Each wave writes its final values
// (g acc, or SiLU(g acc_gate) (g acc_up) with the 32-row gate/up groups; ESZ
// bytes each) into a row-major output tile held in the ring slots the
// exchange used, and the workgroup then writes whole 16-byte pieces of the
// tile's rows to y, instead of one 2- or 4-byte store per accumulator
// element.  Every call issues the same number of stores per wave
// (kEpiStores, what the widest output needs; pieces past the tile, past the
// unit's rows or past the last column go past the buffer and are dropped),
// which the next unit's prefetched loads are counted behind.  A slot holds
// RPS whole rows (a multiple of 4, so the four rows of an accumulator
// register group share a slot); the pieces of a row sit in slot
// c ^ ((row >> 2) & MSK), which spreads the accumulator layout's writes (four
// rows at one column per instruction) over the banks.  The last barrier lets
// the next unit's loads reuse the slots.
template <int BM, int NSLOT, int KW, int BN, int ESZ, bool GLU, int CPOL = 0>
__device__ __forceinline__ void kp_store_tile(const f32x4_t (&out)[BM / 16][BN / KW / 16],
                                              const GemmParams& p, const Unit& u, float gv,
                                              uint8_t* ring, int sl0, int wave, int lane) {
  using L = KpLayout<BM, NSLOT, KW, BN>;
  constexpr int NF = BM / 16, NH = BN / KW / 16;
  constexpr int kSt = L::kEpiStores;
  // opaque copies of the lane and slot indices: otherwise the compiler hoists
  // this epilogue's address arithmetic above the K loop and keeps it live
  // there, in registers the loop needs
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(lane), "+v"(tid), "+s"(sl0), "+s"(wave));
  constexpr int BNO = GLU ? BN / 2 : BN;  // output columns of the tile
  constexpr int RB = BNO * ESZ;           // tile row bytes
  constexpr int CPR = RB / 16;            // 16-byte pieces per row
  constexpr int MSK = (CPR < 16 ? CPR : 16) - 1;
  constexpr int RPS = L::kStage / RB;     // tile rows per ring slot
  static_assert(RPS % 4 == 0 && (BM + RPS - 1) / RPS <= L::kRedSlots, "tile fits the slots");
  static_assert(CPR >= 4 && (CPR & (CPR - 1)) == 0, "row pieces");
  const int nout = GLU ? p.n / 2 : p.n;
  auto row_at = [&](int row) {  // byte address of tile row `row`
    return ((sl0 + row / RPS) % NSLOT) * L::kStage + (row % RPS) * RB;
  };
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int row4 = f * 16 + 4 * q;
    const int base = row_at(row4);
    const int sw = (row4 >> 2) & MSK;
#pragma unroll
    for (int jj = 0; jj < NH; ++jj) {
      if (GLU && (jj & 1)) continue;
      const int col = wave * (NH * 16) + jj * 16 + r16;  // weight row within the unit
      const int ob = (GLU ? (col - r16) / 2 + r16 : col) * ESZ;
      uint8_t* dst = ring + base + ((((ob >> 4) ^ sw)) << 4) + (ob & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v;
        if constexpr (!GLU) {
          v = gv * out[f][jj][r];
        } else {
          const float gate = gv * out[f][jj][r];
          const float up = gv * out[f][(jj + 1) % NH][r];
          // SiLU(gate) = gate / (1 + e^-gate) on the hardware exp2 and
          // reciprocal (relative error ~1e-6, inside the FP32 bound)
          const float e = __builtin_amdgcn_exp2f(-gate * 1.4426950408889634f);
          v = gate * __builtin_amdgcn_rcpf(1.0f + e) * up;
        }
        if constexpr (ESZ == 4) *reinterpret_cast<float*>(dst + r * RB) = v;
        else *reinterpret_cast<uint16_t*>(dst + r * RB) = (uint16_t)float_to_bf16_rne(v);
      }
    }
  }
  __syncthreads();
  const int rows = u.row_end - u.row0;
  const int col_bytes = u.nt * RB;  // first byte of the tile within a row of y
  const int row_bytes = nout * ESZ;
  u32x4_t v[kSt];
  uint32_t off[kSt];
#pragma unroll
  for (int i = 0; i < kSt; ++i) {
    const int ci = tid + i * (KW * 64);
    const int row = ci / CPR, c = ci % CPR;
    v[i] = u32x4_t{0u, 0u, 0u, 0u};
    off[i] = kOffNone;
    if (row < BM) {
      v[i] = *reinterpret_cast<const u32x4_t*>(ring + row_at(row) + ((c ^ ((row >> 2) & MSK)) << 4));
      if (row < rows && col_bytes + 16 * c < row_bytes)
        off[i] = (uint32_t)(row * row_bytes + col_bytes + 16 * c);
    }
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc(static_cast<const char*>(p.y) + (int64_t)u.row0 * row_bytes,
                (uint32_t)(rows * row_bytes));
#pragma unroll
  for (int i = 0; i < kSt; ++i) __builtin_amdgcn_raw_buffer_store_b128(v[i], ry, off[i], 0, CPOL);
}

// The persistent loop of the K-phase kernel over `total` units of product p.
// PH = 0: a plain launch.  PH = 1 / 2: the first / second product of a fused
// gate_up -> down launch (FUSED kernels):
//  - phase 1 stores its output tiles with device-scope (write-through) stores,
//    waits until they have completed and then adds one to its row tile's
//    count in p.rt_counters;
//  - phase 2 reads the first product's output as its activations with
//    device-scope loads, waits (bounded, kp_wait) until its row tile's count
//    covers all n1 column tiles of the first product before the unit's first
//    load (in the previous unit's tail when the unit is prefetched), and takes
//    its global scales from p.g (the schedule's LDS copy holds the first
//    product's).
// The loop for a phase starts with an empty ring (no prefetch across phases).
template <int BM, int NSLOT, int KW, int BN, bool GATHER, int PH>
__device__ __forceinline__ void kp_units(const GemmParams& p, Sched& sc, uint8_t* ring,
                                         int total, int n1, bool& gave_up) {
  using L = KpLayout<BM, NSLOT, KW, BN>;
  constexpr int NF = BM / 16;
  constexpr int NJ = L::kNJ;
  constexpr int NH = NJ / 2;  // column tiles a wave keeps after the K-half exchange
  constexpr int CPS = L::kChunksPerStage;
  constexpr bool P2 = PH == 2;
  constexpr int kEpiCpol = PH == 1 ? kCpolDevice : 0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kp = wave & 1, ch = wave >> 1;
  const int G = gridDim.x;
  // the workgroup's units are snake_unit(round, blockIdx.x, G) for rounds
  // while the unit id is below total (the grid may exceed the unit count of
  // a grouped product, and the map permutes workgroups within a round)
  const int first = snake_unit(0, blockIdx.x, G);
  if (total <= 0 || first >= total) return;
  const KpOffsets<BM, KW, BN> off = kp_offsets<BM, NSLOT, KW, BN>(p.k, wave, lane);
  // the epilogue goes through LDS (a fixed number of 16-byte stores) when
  // there is no K split, the output is addressable by buffer stores and its
  // rows split into whole 16-byte pieces; only then are the next unit's
  // first stages prefetched, behind that fixed store count
  const int nout_bytes = (p.act ? p.n / 2 : p.n) * (p.out_f32 ? 4 : 2);
  const bool can_pf = p.splits == 1 && p.n <= kFixedStoreMaxN && nout_bytes % 16 == 0;
  auto wait_of = [&](const Unit& v) {
    return P2 ? KpWait{p.rt_counters + v.rt, (uint32_t)(n1 + p.wait_extra), p.spin_limit,
                       p.d_status}
              : KpWait{nullptr, 0u, 0, nullptr};
  };
  auto decode = [&](int unit) { return decode_unit<BM, P2>(sc, p, unit, n1); };

  int round = 0;
  Unit u = decode(first);
  KpU cu = kp_unit<BN>(p, u);
  uint32_t cxg[2] = {0u, 0u}, nxg[2] = {0u, 0u};
  if constexpr (GATHER) kp_gather<BM, NSLOT, KW, BN>(cu, cxg, p, u, wave, lane);
  int sb0 = 0, wb0 = 0, pf = 0;
  bool ex = false;
  for (;;) {
    const int nu = snake_unit(round + 1, blockIdx.x, G);
    const bool has_next = nu < total;
    Unit un = u;
    KpU nx = cu;
    if (has_next) {
      un = decode(nu);
      nx = kp_unit<BN>(p, un);
      if constexpr (GATHER) kp_gather<BM, NSLOT, KW, BN>(nx, nxg, p, un, wave, lane);
    }
    const int pn = (has_next && can_pf && cu.nch >= NSLOT) ? min(L::kPrefetch, nx.nch) : 0;
    // a unit whose first stages were not prefetched waits here for its
    // activations (a prefetched one waited before its first load)
    if (P2 && pf == 0) kp_wait(wait_of(u), gave_up);
    const float gv = P2 ? __uint_as_float(sload_u32(p.g, 4u * (uint32_t)u.e)) : expert_g(p, u.e);
    // 16-row fragments holding rows of this tile (the rest is padding)
    const int nf = min(NF, (u.row_end - u.row0 + 15) / 16);
    const KpWait nxw = wait_of(un);

    f32x4_t acc[NF][NJ];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#define NVFP4_KLOOP(NFE)                                                                        \
  kp_kloop<BM, NSLOT, KW, BN, NFE, GATHER, P2>(acc, ring, cu, sb0, wb0, pf, ex, nx, pn,         \
                                               cxg[0], cxg[1], nxg[0], nxg[1], off, kp, ch,     \
                                               wave, lane, nxw, gave_up)
    switch (nf) {
      case 1: NVFP4_KLOOP(1); break;
      case 2: NVFP4_KLOOP(NF >= 2 ? 2 : NF); break;
      case 3: NVFP4_KLOOP(NF >= 3 ? 3 : NF); break;
      default: NVFP4_KLOOP(NF); break;
    }
#undef NVFP4_KLOOP

    // Sum the two K halves: wave w keeps column tiles [NH kp, NH kp + NH) of
    // its NJ and hands the others to wave w ^ 1 through 1 KB chunks in the
    // ring slots not holding the next unit's first stages.
    __syncthreads();
    auto chunk = [&](int k) {
      const int sl = (sb0 + cu.nch + pn + k / CPS) % NSLOT;
      return reinterpret_cast<f32x4_t*>(ring + sl * L::kStage + (k % CPS) * 1024) + lane;
    };
    f32x4_t out[NF][NH];
    // (the branch is wave-uniform; both sides index the accumulators with
    // constants so they stay in registers)
    if (kp == 0) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj) *chunk(wave * (NF * NH) + f * NH + jj) = acc[f][NH + jj];
      __syncthreads();
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj)
          out[f][jj] = acc[f][jj] + *chunk((wave ^ 1) * (NF * NH) + f * NH + jj);
    } else {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj) *chunk(wave * (NF * NH) + f * NH + jj) = acc[f][jj];
      __syncthreads();
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj)
          out[f][jj] = *chunk((wave ^ 1) * (NF * NH) + f * NH + jj) + acc[f][NH + jj];
    }
    __syncthreads();  // exchange chunks read before the next unit's loads reuse them
    // wave w now owns columns [w CPW/2, (w + 1) CPW/2) of the unit
    if (can_pf) {
      const int sl0 = (sb0 + cu.nch + pn) % NSLOT;
      if (p.act) {
        if (p.out_f32)
          kp_store_tile<BM, NSLOT, KW, BN, 4, true, kEpiCpol>(out, p, u, gv, ring, sl0, wave, lane);
        else
          kp_store_tile<BM, NSLOT, KW, BN, 2, true, kEpiCpol>(out, p, u, gv, ring, sl0, wave, lane);
      } else {
        if (p.out_f32)
          kp_store_tile<BM, NSLOT, KW, BN, 4, false, kEpiCpol>(out, p, u, gv, ring, sl0, wave, lane);
        else
          kp_store_tile<BM, NSLOT, KW, BN, 2, false, kEpiCpol>(out, p, u, gv, ring, sl0, wave, lane);
      }
    } else {
      finish_tile<NF, NH, KW, BN>(out, p, u, gv, sc);
    }
    if constexpr (PH == 1) {
      // the tile's stores have completed (write-through, device scope) before
      // its row tile's count goes up; the wait also covers the next unit's
      // prefetched loads, which were issued earlier
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(p.rt_counters + u.rt, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!has_next) break;
    sb0 = (sb0 + cu.nch) % NSLOT;
    wb0 = (wb0 + (cu.nch + L::kWinStages - 1) / L::kWinStages) % L::kWinBufs;
    pf = pn;
    ex = pn > 0;
    u = un;
    cu = nx;
    cxg[0] = nxg[0];
    cxg[1] = nxg[1];
    ++round;
  }
}

// GATHER: activation rows come through p.row_index (see kp_gather).
// FUSED: p is a fused gate_up -> down launch (its second product in p.w2 ...),
// run as two phases of one persistent loop each.
template <int BM, int NSLOT, int KW, int BN, bool GATHER = false, bool FUSED = false>
__global__ __launch_bounds__(KW * 64) void gemm_kp_kernel(GemmParams p) {
  static_assert(kp_fits_lds<BM, NSLOT, KW, BN>(), "LDS budget");
  static_assert(!(GATHER && FUSED), "fused launches read pre-permuted rows");
  __shared__ __attribute__((aligned(16))) uint8_t ring[KpLayout<BM, NSLOT, KW, BN>::kTotal];
  __shared__ Sched sc;
  const int total = build_schedule<KW * 64, BM>(sc, p);
  bool gave_up = false;
  if constexpr (!FUSED) {
    kp_units<BM, NSLOT, KW, BN, GATHER, 0>(p, sc, ring, total, 1, gave_up);
  } else {
    if (total <= 0) return;
    kp_units<BM, NSLOT, KW, BN, false, 1>(p, sc, ring, total, 1, gave_up);
    // the second product: h = the first product's output as activations;
    // its schedule is the first's (same experts and row tiles), scaled
    __syncthreads();  // every wave is done with the ring
    GemmParams q = p;
    q.x = static_cast<const uint16_t*>(p.y);
    q.w = p.w2;
    q.s = p.s2;
    q.g = p.g2;
    q.y = p.y2;
    q.n = p.n2;
    q.k = p.k2;
    q.k_split = p.k2;
    q.n_tiles = p.n_tiles2;
    q.out_f32 = p.out2_f32;
    q.act = 0;
    const int total2 = total / p.n_tiles * p.n_tiles2;
    kp_units<BM, NSLOT, KW, BN, false, 2>(q, sc, ring, total2, p.n_tiles, gave_up);
  }
}

// ---- large-M kernel (k % 64 == 0, many rows) -----------------------------------
//
// For a dense product with at least a few hundred rows a 256 x 256 output
// tile per workgroup of 8 waves amortizes the activation and weight traffic:
// wave w computes all 256 rows x columns [32 w, 32 w + 32) of the tile as
// 8 x 1 v_mfma_f32_32x32x16_bf16 tiles (FP32 accumulators), so every weight
// of the tile is dequantized by one wave only (two waves sharing a column
// range, each on half of the rows, both dequantized it: 2-4 % slower at
// 8192^3), at the price of reading each activation fragment from LDS in all
// eight waves.  Two waves share each SIMD, so one wave's dequantization and
// load issue run while the other's MFMAs occupy the matrix pipeline.  K advances in 64-wide steps.  LDS holds a 4-slot ring of
// activation tiles (256 rows x 128 B), a 3-slot ring of packed weight tiles
// (256 rows x 32 B, only the 4.5-bit data) and two windows of block scales
// covering 4 steps each (256 rows x 16 B, one 16-byte load per row: a load
// per row and step of 4 bytes cost 6 % of the launch).  During step s
// (between its MFMA sub-steps, so the load path works while the matrix pipe
// does) the weights of step s + 2 (with the scale window that starts there)
// and the activations of step s + 3 are issued, and the barrier at the top
// of step s waits only for step s's own loads.  Every workgroup of an XCD reads the same activation rows at about
// the same time, so each activation step is in effect a miss to HBM for all
// of them; three steps of lead hide that latency where two did not (8192^3:
// 941 -> 848 us in a timing copy).  Weight lines (128 B = four steps of a
// row) miss once in four steps, and two steps of lead cover them.  Each wave
// dequantizes its own 32 columns of the step from the packed bytes in
// registers, which keeps BF16 weights out of LDS.
//
// K slots: in sub-step ks (16 K) of a step, lane l (row / column l % 32,
// half h = l / 32) supplies K = 32 h + 8 ks .. + 7 of the step, for both
// operands (the MFMA sums over its 16 K slots in any assignment as long as A
// and B agree).  So a lane's weight bytes for the whole step are 16
// contiguous bytes of its column, and each dword of them is one sub-step.
// LDS rows of the activation tile keep their 16-byte chunk c in slot
// c ^ ((r >> 1) & 7), so the 32-row fragment reads spread over all banks.
constexpr int kLmBM = 256, kLmBN = 256, kLmBK = 64;
// waves per workgroup split as kLmWM row groups x kLmWN column groups
constexpr int kLmWN = 8, kLmWM = 8 / kLmWN;
constexpr int kLmRW = kLmBM / kLmWM, kLmCW = kLmBN / kLmWN;  // rows, columns per wave
constexpr int kLmNI = kLmRW / 32, kLmNJ = kLmCW / 32;         // 32 x 32 tiles per wave

struct LmLayout {
  static constexpr int kWaves = 8;
  static constexpr int kXSlots = 4;                          // activation steps ahead: 3
  static constexpr int kWSlots = 3;                          // weight steps ahead: 2
  static constexpr int kXStage = kLmBM * kLmBK * 2;          // 32 KB
  static constexpr int kWpStage = kLmBN * kLmBK / 2;         // 8 KB
  static constexpr int kWinSteps = 4;                        // steps per scale window
  static constexpr int kWinBytes = kLmBN * kWinSteps * 4;    // 4 KB: 16 B per weight row
  static constexpr int kW = kXSlots * kXStage;               // first packed weight slot
  static constexpr int kWin = kW + kWSlots * kWpStage;       // first scale window
  static constexpr int kTotal = kWin + 2 * kWinBytes;        // 160 KB
  static constexpr int kXLoads = kXStage / 1024 / kWaves;    // per wave per step: 4
  static constexpr int kWpLoads = kWpStage / 1024 / kWaves;  // per wave per step: 1
  static constexpr int kWinLoads = kWinBytes / 1024;         // waves 0..3, one each
  static constexpr int kEpiBytes = 32 * 32 * 4;              // per wave: one FP32 32 x 32 tile
  static_assert(kTotal <= 160 * 1024, "LDS budget");
  static_assert(kXLoads == 4 && kWpLoads == 1 && kWinLoads <= kWaves, "load split");
  static_assert(kWaves * kEpiBytes <= kW, "epilogue scratch");
};

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ int lm_swz(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

struct LmOffsets {
  uint32_t x[LmLayout::kXLoads];
  uint32_t wp;
  uint32_t s;
};

__device__ __forceinline__ LmOffsets lm_offsets(int K, int wave, int lane) {
  LmOffsets o;
  // activations: load t covers tile rows 8t..8t+7 (128 B each); slot c of
  // row r receives chunk c ^ ((r >> 1) & 7)
#pragma unroll
  for (int tt = 0; tt < LmLayout::kXLoads; ++tt) {
    const int r = (wave * LmLayout::kXLoads + tt) * 8 + (lane >> 3);
    const int g = (lane & 7) ^ ((r >> 1) & 7);
    o.x[tt] = (uint32_t)r * (uint32_t)(K * 2) + (uint32_t)(16 * g);
  }
  // packed weights: wave w loads rows 32w..32w+31 (32 B each, unswizzled)
  o.wp = (uint32_t)(wave * 32 + (lane >> 1)) * (uint32_t)(K / 2) + (uint32_t)(16 * (lane & 1));
  // scale window: wave w < 4 loads rows 64w..64w+63, 16 B (4 steps) each
  o.s = (uint32_t)((wave & 3) * 64 + lane) * (uint32_t)(K / 16);
  return o;
}

// The packed weights of a step into its weight slot, preceded (every
// kWinSteps-th step, waves 0..3) by the scale window that starts there.
__device__ __forceinline__ void lm_issue_w(uint32_t ring0, int step, u32x4_t rw, u32x4_t rs,
                                           const LmOffsets& o, int wave) {
  using L = LmLayout;
  if (step % L::kWinSteps == 0 && wave < L::kWinLoads)
    lds_dma16(ring0 + L::kWin + ((step / L::kWinSteps) & 1) * L::kWinBytes + wave * 1024, o.s,
              (uint32_t)(step * kLmBK / 16), rs);
  lds_dma16(ring0 + L::kW + (uint32_t)((step % L::kWSlots) * L::kWpStage) + wave * 1024, o.wp,
            (uint32_t)(step * kLmBK / 2), rw);
}

// Load tt (of four) of a step's activations into its slot.
__device__ __forceinline__ void lm_issue_x(uint32_t ring0, int step, int tt, u32x4_t rx,
                                           const LmOffsets& o, int wave) {
  const uint32_t st = ring0 + (uint32_t)((step % LmLayout::kXSlots) * LmLayout::kXStage);
  lds_dma16(st + (wave * LmLayout::kXLoads + tt) * 1024, o.x[tt], (uint32_t)(step * kLmBK * 2), rx);
}

// Activation fragments of sub-step ks: the row tiles of the wave's rows.
__device__ __forceinline__ void lm_read_a(bf16x8_t (&a)[kLmNI], const uint8_t* st, int ks, int wm,
                                          int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < kLmNI; ++i)
    a[i] = *reinterpret_cast<const bf16x8_t*>(st + lm_swz(wm * kLmRW + i * 32 + r32, 4 * h + ks));
}

// Dense only (offsets == nullptr, one expert): tile t of the grid is
// (row tile t / n_tiles, column tile t % n_tiles) after an XCD-aware remap.
__global__ __launch_bounds__(LmLayout::kWaves * 64) void gemm_lm_kernel(GemmParams p) {
  using L = LmLayout;
  __shared__ __attribute__((aligned(16))) uint8_t ring[L::kTotal];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kLmWN, wn = wave % kLmWN;  // row group, column group
  const int r32 = lane & 31, h = lane >> 5;
  const int N = p.n, K = p.k;
  const int m_tiles = (int)((p.rows + kLmBM - 1) / kLmBM);
  const int total = m_tiles * p.n_tiles;
  const uint32_t ring0 = lds_addr(ring);
  const LmOffsets off = lm_offsets(K, wave, lane);
  const int nsteps = K / kLmBK;
  const float gv = p.g[0];
  const int ob = p.out_f32 ? 4 : 2;
  // the epilogue writes whole 16-column pieces of rows when every piece is
  // 16-byte aligned, none straddles the last column and a tile's rows stay
  // inside one 32-bit buffer range
  const bool vec_out = N % 16 == 0 && (int64_t)kLmBM * N * ob < ((int64_t)1 << 31);
  // the lane's weight bytes within a weight slot and its scales within a
  // window, per column tile j
  uint32_t wp_at[kLmNJ], s_at[kLmNJ];
#pragma unroll
  for (int j = 0; j < kLmNJ; ++j) {
    wp_at[j] = (uint32_t)((wn * kLmCW + j * 32 + r32) * 32 + 16 * h);
    s_at[j] = (uint32_t)((wn * kLmCW + j * 32 + r32) * 16);
  }

  for (int round = 0; round * (int)gridDim.x < total; ++round) {
    const int t = round_unit(round, blockIdx.x, gridDim.x);
    if (t >= total) continue;
    const int mt = t / p.n_tiles, nt = t % p.n_tiles;
    const int row0 = mt * kLmBM, n0 = nt * kLmBN;
    const int row_end = (int)min((int64_t)row0 + kLmBM, p.rows);
    const u32x4_t rx = rsrc_words(p.x + (int64_t)row0 * K, (uint32_t)(row_end - row0) * (uint32_t)(K * 2));
    const u32x4_t rw = rsrc_words(p.w + (int64_t)n0 * (K / 2),
                                  (uint32_t)(min(N - n0, kLmBN)) * (uint32_t)(K / 2));
    const u32x4_t rs = rsrc_words(p.s + (int64_t)n0 * (K / 16),
                                  (uint32_t)(min(N - n0, kLmBN)) * (uint32_t)(K / 16));

    f32x16_t acc[kLmNI][kLmNJ];
#pragma unroll
    for (int i = 0; i < kLmNI; ++i)
#pragma unroll
      for (int j = 0; j < kLmNJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // The issue order is that of steady state from virtual step -3 on: in
    // step v, the weights of step v + 2, then the activations of step v + 3.
    // So after the weights of step s come the activations of step s + 1 and
    // the weights of step s + 1 (at least 5 loads per wave, if step s + 1
    // exists) and the activations of step s + 2 (4, if it exists); the
    // activations of step s went out before the weights of step s.  (A scale
    // window among the weights of step s + 1 makes the wait below cover one
    // load more than it must.)
#pragma unroll
    for (int tt = 0; tt < L::kXLoads; ++tt) lm_issue_x(ring0, 0, tt, rx, off, wave);
    for (int v = 0; v < 2; ++v) {
      if (v < nsteps) lm_issue_w(ring0, v, rw, rs, off, wave);
      if (v + 1 < nsteps) {
#pragma unroll
        for (int tt = 0; tt < L::kXLoads; ++tt) lm_issue_x(ring0, v + 1, tt, rx, off, wave);
      }
    }
    for (int s = 0; s < nsteps; ++s) {
      // this wave's loads of step s are done; the barrier makes every
      // wave's done, and every wave is past step s - 1, whose slots the
      // loads issued in this step take
      if (s + 2 < nsteps) wait_vmcnt_c<L::kXLoads + L::kWpLoads + L::kXLoads>();
      else if (s + 1 < nsteps) wait_vmcnt_c<L::kXLoads + L::kWpLoads>();
      else wait_vmcnt_c<0>();
      __syncthreads();
      const uint8_t* st = ring + (s % L::kXSlots) * L::kXStage;
      const uint8_t* wst = ring + L::kW + (s % L::kWSlots) * L::kWpStage;
      const uint8_t* win = ring + L::kWin + ((s / L::kWinSteps) & 1) * L::kWinBytes +
                           4 * (s % L::kWinSteps);
      const bool prew = s + 2 < nsteps, prex = s + 3 < nsteps;
      u32x4_t wd[kLmNJ];
      uint32_t sc[kLmNJ];
#pragma unroll
      for (int j = 0; j < kLmNJ; ++j) {
        wd[j] = *reinterpret_cast<const u32x4_t*>(wst + wp_at[j]);
        sc[j] = *reinterpret_cast<const uint32_t*>(win + s_at[j]) >> (16 * h);
      }
      bf16x8_t a[2][kLmNI], b[2][kLmNJ];
      lm_read_a(a[0], st, 0, wm, lane);
#pragma unroll
      for (int j = 0; j < kLmNJ; ++j) b[0][j] = dequant8(wd[j][0], decode_e4m3<0>(sc[j]));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks + 1 < 4) lm_read_a(a[(ks + 1) & 1], st, ks + 1, wm, lane);
#pragma unroll
        for (int i = 0; i < kLmNI; ++i)
#pragma unroll
          for (int j = 0; j < kLmNJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 1][i], b[ks & 1][j],
                                                                acc[i][j], 0, 0, 0);
        if (ks + 1 < 4) {
#pragma unroll
          for (int j = 0; j < kLmNJ; ++j)
            b[(ks + 1) & 1][j] = dequant8(wd[j][ks + 1], ((ks + 1) >> 1) ? decode_e4m3<1>(sc[j])
                                                                         : decode_e4m3<0>(sc[j]));
        }
        // one activation load per sub-step (bunched, they held the wave
        // longer at the load path)
        if (ks == 0 && prew) lm_issue_w(ring0, s + 2, rw, rs, off, wave);
        if (prex) lm_issue_x(ring0, s + 3, ks, rx, off, wave);
      }
    }
    __syncthreads();  // every wave's fragment reads done: the ring is free

    if (vec_out) {
      // epilogue through a per-wave 32 x 32 FP32 scratch tile: lane l of
      // tile (i, j) holds column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4;
      // read back, lane l takes row l / 2, columns 16 (l % 2) .. + 15, and
      // writes them as whole 16-byte pieces
      float* scr = reinterpret_cast<float*>(ring + wave * L::kEpiBytes);
      const int rr = lane >> 1, hh = lane & 1;
      const int row_bytes = N * ob;
      const __amdgpu_buffer_rsrc_t ry =
          make_rsrc(static_cast<const char*>(p.y) + (int64_t)row0 * row_bytes,
                    (uint32_t)((row_end - row0) * row_bytes));
#pragma unroll
      for (int i = 0; i < kLmNI; ++i)
#pragma unroll
        for (int j = 0; j < kLmNJ; ++j) {
#pragma unroll
          for (int e = 0; e < 16; ++e) scr[(8 * (e >> 2) + 4 * h + (e & 3)) * 32 + r32] = acc[i][j][e];
          f32x4_t v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            v[c] = *reinterpret_cast<const f32x4_t*>(scr + rr * 32 + 16 * hh + 4 * c);
          const int row = wm * kLmRW + i * 32 + rr;  // within the tile
          const int col = n0 + wn * kLmCW + j * 32 + 16 * hh;
          const bool ok = row0 + row < row_end && col < N;
          const uint32_t o = ok ? (uint32_t)(row * row_bytes + col * ob) : kOffNone;
          if (p.out_f32) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              __builtin_amdgcn_raw_buffer_store_b128(
                  __builtin_bit_cast(u32x4_t, f32x4_t{gv * v[c][0], gv * v[c][1], gv * v[c][2],
                                                      gv * v[c][3]}),
                  ry, o + (ok ? 16 * c : 0), 0, 0);
          } else {
            uint32_t w[8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              w[2 * c] = float_to_bf16_rne(gv * v[c][0]) | (float_to_bf16_rne(gv * v[c][1]) << 16);
              w[2 * c + 1] = float_to_bf16_rne(gv * v[c][2]) | (float_to_bf16_rne(gv * v[c][3]) << 16);
            }
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{w[0], w[1], w[2], w[3]}, ry, o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{w[4], w[5], w[6], w[7]}, ry,
                                                   o + (ok ? 16 : 0), 0, 0);
          }
        }
      __syncthreads();  // scratch reads done before the next tile's loads land
    } else {
      // lane l of tile (i, j) holds column l % 32 and rows
      // 8 (e / 4) + 4 (l / 32) + e % 4 of the 32 x 32 block
#pragma unroll
      for (int i = 0; i < kLmNI; ++i)
#pragma unroll
        for (int j = 0; j < kLmNJ; ++j) {
          const int col = n0 + wn * kLmCW + j * 32 + r32;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = row0 + wm * kLmRW + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            if (row < row_end && col < N) {
              const float v = gv * acc[i][j][e];
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
}

// ---- register kernel (any k % 16 == 0) ------------------------------------------

constexpr int kRegThreads = 256;   // 4 waves
constexpr int kRegWaves = kRegThreads / kWave;
constexpr int kNW = 4;             // MFMA column tiles per wave
constexpr int kKC = 256;           // K per chunk
constexpr int kRegBN = kRegWaves * kNW * 16;  // columns per unit (256)
constexpr int kLdsStride = kKC + 8;  // BF16 elements per staged activation row (16 B pad)

// One lane's packed weights (8 dwords = 64 nibbles along K) and its 4 block
// scales for each of the wave's kNW column tiles, for one 256-wide K chunk.
struct WTile {
  uint32_t w[kNW][8];
  uint32_t s[kNW];
};

__device__ __forceinline__ void load_wtile(WTile& t, __amdgpu_buffer_rsrc_t rw,
                                           __amdgpu_buffer_rsrc_t rs, const int (&nrow)[kNW],
                                           int K, int kpos, int k_end) {
#pragma unroll
  for (int j = 0; j < kNW; ++j) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kd = kpos + 8 * u;
      const uint32_t o = kd < k_end ? (uint32_t)nrow[j] * (uint32_t)(K / 2) + (uint32_t)(kd / 2)
                                    : kOffNone;
      t.w[j][u] = __builtin_amdgcn_raw_buffer_load_b32(rw, o, 0, 0);
    }
    uint32_t sv = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int kb = kpos + 16 * b;
      const uint32_t o = kb < k_end ? (uint32_t)nrow[j] * (uint32_t)(K / 16) + (uint32_t)(kb / 16)
                                    : kOffNone;
      sv |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, o, 0, 0) << (8 * b);
    }
    t.s[j] = sv;
  }
}

// Activation chunk [row0, row0 + BM) x [kc, kc + 256): 16-byte pieces, one
// per thread per pass, zero outside the segment / split.
template <int BM>
__device__ __forceinline__ void load_xtile(u32x4_t (&xr)[BM / 8], const GemmParams& p,
                                           int row0, int row_end, int K, int kc, int k_end,
                                           int tid) {
#pragma unroll
  for (int pass = 0; pass < BM / 8; ++pass) {
    const int pc = tid + kRegThreads * pass;
    const int grow = row0 + (pc >> 5);
    const int kk = kc + (pc & 31) * 8;
    xr[pass] = u32x4_t{0u, 0u, 0u, 0u};
    if (grow < row_end && kk < k_end) {
      // routed row grow reads token row row_index[grow] when an index is given
      int64_t xrow = grow;
      if (p.row_index != nullptr) {
        const uint32_t tok = (uint32_t)p.row_index[grow];
        if (tok >= (uint32_t)p.x_rows) {
          if (kk == kc && p.d_status != nullptr) atomicOr(p.d_status, NVFP4_DSTATUS_BAD_INDEX);
          continue;
        }
        xrow = tok;
      }
      xr[pass] = *reinterpret_cast<const u32x4_t*>(p.x + xrow * K + kk);
    }
  }
}

template <int BM>
__device__ __forceinline__ void store_xtile(uint16_t* xs, const u32x4_t (&xr)[BM / 8], int tid) {
#pragma unroll
  for (int pass = 0; pass < BM / 8; ++pass) {
    const int pc = tid + kRegThreads * pass;
    *reinterpret_cast<u32x4_t*>(&xs[(pc >> 5) * kLdsStride + (pc & 31) * 8]) = xr[pass];
  }
}

// 8 MFMA steps of 32 K slots over one staged chunk; lane group q supplies
// K = kc + 64q + 8i .. +7 in step i.
template <int BM>
__device__ __forceinline__ void reg_compute(f32x4_t (&acc)[BM / 16][kNW], const uint16_t* xs,
                                            const WTile& t, int q, int r16) {
  constexpr int NF = BM / 16;
  float scl[kNW][4];
#pragma unroll
  for (int j = 0; j < kNW; ++j) {
    scl[j][0] = decode_e4m3<0>(t.s[j]);
    scl[j][1] = decode_e4m3<1>(t.s[j]);
    scl[j][2] = decode_e4m3<2>(t.s[j]);
    scl[j][3] = decode_e4m3<3>(t.s[j]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16x8_t a[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
      a[f] = *reinterpret_cast<const bf16x8_t*>(&xs[(f * 16 + r16) * kLdsStride + 64 * q + 8 * i]);
#pragma unroll
    for (int j = 0; j < kNW; ++j) {
      const bf16x8_t b = dequant8(t.w[j][i], scl[j][i >> 1]);
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f], b, acc[f][j], 0, 0, 0);
    }
  }
}

template <int BM>
__global__ __launch_bounds__(kRegThreads) void gemm_reg_kernel(GemmParams p) {
  constexpr int NF = BM / 16;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kLdsStride];
  __shared__ Sched sc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int total = build_schedule<kRegThreads, BM>(sc, p);
  const int N = p.n, K = p.k;

  for (int round = 0; round * (int)gridDim.x < total; ++round) {
    const int unit = round_unit(round, blockIdx.x, gridDim.x);
    if (unit >= total) continue;
    const Unit u = decode_unit<BM>(sc, p, unit);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(p.w + (int64_t)u.e * N * (K / 2), (uint32_t)N * (uint32_t)(K / 2));
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(p.s + (int64_t)u.e * N * (K / 16), (uint32_t)N * (uint32_t)(K / 16));
    int nrow[kNW];
#pragma unroll
    for (int j = 0; j < kNW; ++j) nrow[j] = u.nt * kRegBN + wave * (kNW * 16) + j * 16 + r16;

    f32x4_t acc[NF][kNW];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < kNW; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // two-stage pipeline: chunk c+1's weights (registers) and activations
    // (registers, then LDS) are in flight while chunk c is multiplied out
    const int nch = (u.k_end - u.k_beg + kKC - 1) / kKC;
    WTile wa, wb;
    u32x4_t xr[BM / 8];
    load_wtile(wa, rw, rs, nrow, K, u.k_beg + 64 * q, u.k_end);
    load_xtile<BM>(xr, p, u.row0, u.row_end, K, u.k_beg, u.k_end, tid);
    store_xtile<BM>(xs[0], xr, tid);
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {
      const int kc = u.k_beg + c * kKC;
      const bool more1 = c + 1 < nch;
      if (more1) {
        load_wtile(wb, rw, rs, nrow, K, kc + kKC + 64 * q, u.k_end);
        load_xtile<BM>(xr, p, u.row0, u.row_end, K, kc + kKC, u.k_end, tid);
      }
      reg_compute<BM>(acc, xs[0], wa, q, r16);
      if (more1) store_xtile<BM>(xs[1], xr, tid);
      __syncthreads();
      if (!more1) break;
      const bool more2 = c + 2 < nch;
      if (more2) {
        load_wtile(wa, rw, rs, nrow, K, kc + 2 * kKC + 64 * q, u.k_end);
        load_xtile<BM>(xr, p, u.row0, u.row_end, K, kc + 2 * kKC, u.k_end, tid);
      }
      reg_compute<BM>(acc, xs[1], wb, q, r16);
      if (more2) store_xtile<BM>(xs[0], xr, tid);
      __syncthreads();
    }
    finish_tile<NF, kNW, kRegWaves, kRegBN>(acc, p, u, expert_g(p, u.e), sc);
  }
}

// ---- host side -----------------------------------------------------------------

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

template <typename KernelT>
static int occupancy_of(KernelT kernel, int threads, int dyn_lds) {
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, dyn_lds) != hipSuccess ||
      v < 1)
    v = 1;
  return v;
}

static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

// Kernel configuration of a plan (GemmPlan::kind):
//   0  register kernel, 4 waves x 256 columns (any k % 16 == 0)
//   1  K-phase kernel, 4 waves x 128 columns, two workgroups per CU (tiles of
//      up to 32 rows)
//   2  K-phase kernel, 8 waves x 256 columns (64-row tiles, or any tile size
//      with NVFP4_KPCFG=8)
//   3  large-M kernel, 256 x 256 tiles (dense products with at least
//      kLmMinRows rows; NVFP4_LM=0 disables it)
//   4  K-phase kernel, 4 waves x 64 columns (dense, up to 16 rows)
//   6  dot-product kernel (dense, one to six rows; gemv.hip)
//   7  one MFMA row tile per 16 columns, whole K (dense, 5 and 6 rows whose
//      K is too long for kind 6, and 7 to 16 rows with NVFP4_DSK=0 or where
//      kind 8's counters cannot hold the column tiles; gemv.hip)
//   8  split-K decode kernel, 64 columns per unit (dense, 7 to 64 rows, or
//      5 to 64 with NVFP4_DSK=2; NVFP4_DSK=0 disables it; gemv.hip)
constexpr int kLmMinRows = 256;
constexpr int kMinSplitStages = 7;

static void choose_kernel(GemmPlan& pl, int64_t rows, int64_t n, int64_t k, bool grouped,
                          int cu_count) {
  // the large-M kernel has no K split: it needs a 256 x 256 output tile for
  // every CU (at N = 4096, K = 7168 it is 1.2-5x slower than the 64-row
  // K-phase kernel with split K from 256 to 2048 rows, and faster at 4096)
  const int64_t lm_tiles = ((rows + kLmBM - 1) / kLmBM) * ((n + kLmBN - 1) / kLmBN);
  const int lm = env_int("NVFP4_LM", 1);  // 0: never, 2: whenever the shape allows
  // (its buffer offsets address a 256-row activation tile in 31 bits)
  const bool lm_fits = (int64_t)kLmBM * 2 * k < ((int64_t)1 << 31);
  if (pl.fast && !grouped && rows >= kLmMinRows && lm != 0 && lm_fits &&
      (lm == 2 || lm_tiles >= cu_count)) {
    pl.kind = 3; pl.bn = kLmBN; pl.bm = kLmBM;
  } else if (!pl.fast) {
    pl.kind = 0; pl.bn = 256; pl.nslot = 0;
  } else if (!grouped && pl.bm == 16 && env_int("NVFP4_KPCFG", 64) == 64) {
    // dense decode (up to 16 rows): 64-column tiles, three workgroups per CU,
    // twice the units of 128-column tiles at the same K split (6-8 % faster
    // at N = 4096, K = 7168); each wave keeps one column tile after the
    // K-half exchange, so this never serves the SiLU(gate) * up epilogue
    pl.kind = 4; pl.bn = 64; pl.nslot = 5;
  } else if (pl.bm <= 32 && env_int("NVFP4_KPCFG", 4) != 8) {
    pl.kind = 1; pl.bn = 128; pl.nslot = pl.bm == 16 ? 5 : 4;
  } else {
    pl.kind = 2; pl.bn = 256; pl.nslot = pl.bm == 64 ? 4 : 5;
  }
}

// Resident workgroups per CU of the chosen kernel with its dynamic LDS
// (cached per kernel and 256-byte step of the schedule size).
static int occupancy_for(const GemmPlan& pl) {
  constexpr int kSteps = kSchedLdsMax / 256 + 2;
  static std::atomic<int> cache[5][3][kSteps];
  static std::once_flag once;
  std::call_once(once, [] {
    for (auto& a : cache)
      for (auto& b : a)
        for (auto& c : b) c.store(-1);
  });
  const int bi = pl.bm == 16 ? 0 : (pl.bm == 32 ? 1 : 2);
  const int dyn = pl.dyn_lds;
  std::atomic<int>& slot = cache[pl.kind][bi][std::min(kSteps - 1, (dyn + 255) / 256)];
  int c = slot.load();
  if (c < 0) {
    if (pl.kind == 0) {
      c = pl.bm == 16 ? occupancy_of(gemm_reg_kernel<16>, kRegThreads, dyn)
          : pl.bm == 32 ? occupancy_of(gemm_reg_kernel<32>, kRegThreads, dyn)
                        : occupancy_of(gemm_reg_kernel<64>, kRegThreads, dyn);
    } else if (pl.kind == 3) {
      c = occupancy_of(gemm_lm_kernel, LmLayout::kWaves * 64, dyn);
    } else if (pl.kind == 1) {
      c = pl.bm == 16 ? occupancy_of(gemm_kp_kernel<16, 5, 4, 128>, 256, dyn)
                      : occupancy_of(gemm_kp_kernel<32, 4, 4, 128>, 256, dyn);
    } else if (pl.kind == 4) {
      c = occupancy_of(gemm_kp_kernel<16, 5, 4, 64>, 256, dyn);
    } else {
      c = pl.bm == 16 ? occupancy_of(gemm_kp_kernel<16, 5, 8, 256>, 512, dyn)
          : pl.bm == 32 ? occupancy_of(gemm_kp_kernel<32, 5, 8, 256>, 512, dyn)
                        : occupancy_of(gemm_kp_kernel<64, 4, 8, 256>, 512, dyn);
    }
    slot.store(c);
  }
  return c;
}

GemmPlan plan_gemm(int64_t rows, int64_t num_experts, int64_t n, int64_t k, bool grouped,
                   int cu_count, bool allow_split) {
  GemmPlan pl{};
  pl.fast = (k % 64) == 0;
  // one to six dense rows: the dot-product kernel, 16 columns per workgroup,
  // whole K, no workspace (kind 6).  At N = 4096, K = 7168 it takes 8.2 /
  // 9.1 us at 5 / 6 rows against 9.3 / 9.6 us for kind 7
  // NVFP4_DSK=2 (tuning): the split-K decode kernel from five rows
  const int dsk = env_int("NVFP4_DSK", 1);
  const int gemv_rows = dsk == 2 ? 4 : kGemvMaxRows;
  if (!grouped && rows >= 1 && rows <= gemv_rows && k % 32 == 0 &&
      rows * k * 2 <= kGemvMaxXBytes && env_int("NVFP4_GEMV", 1) != 0) {
    pl.kind = 6;
    pl.bm = (int)rows;
    pl.bn = 16;
    pl.splits = 1;
    pl.k_split = (int)k;
    pl.n_tiles = (int)((n + 15) / 16);
    pl.max_tiles = pl.n_tiles;
    pl.grid = pl.n_tiles;
    pl.dyn_lds = (int)(rows * k * 2);
    pl.ws_bytes = 0;
    return pl;
  }
  // 7 to 64 dense rows, k % 128 == 0: split-K decode kernel, 64 columns per
  // unit, each workgroup's weight share in flight at once (kind 8,
  // gemv.hip); the split count about fills the CUs with units.  At N = 4096,
  // K = 7168 it takes 9.6 / 9.6 / 9.7 / 11.2 / 14.0 / 15.7 us at 7 / 12 / 16 /
  // 32 / 48 / 64 rows, against 10.0 us for kind 7 at 7 and 8 rows and 17.3 /
  // 19-20 / 20 us for the K-phase kernel at 32 / 48 / 64 rows
  // (rows of five and six reach here only when the dot-product kernel cannot
  // stage them: a long K, or NVFP4_DSK=2)
  if (!grouped && rows > 4 && rows <= 64 && k % 128 == 0 && env_int("NVFP4_GEMV", 1) != 0 &&
      (dsk == 2 || (dsk == 1 && rows > 6))) {
    const int64_t n_tiles = (n + kDskCols - 1) / kDskCols;
    const int64_t groups = k / 128;
    int64_t splits = std::min<int64_t>(groups, std::max<int64_t>(1, cu_count / n_tiles));
    splits = std::max<int64_t>(splits, (groups + kDskMaxGroups - 1) / kDskMaxGroups);
    const int64_t kgroups = (groups + splits - 1) / splits;
    splits = (groups + kgroups - 1) / kgroups;
    if (splits == 1 || n_tiles <= kMaxCounters) {
      pl.kind = 8;
      pl.bm = (int)((rows + 15) / 16 * 16);
      pl.bn = kDskCols;
      pl.splits = (int)splits;
      pl.k_split = (int)(kgroups * 128);
      pl.n_tiles = (int)n_tiles;
      pl.max_tiles = pl.n_tiles;
      pl.grid = (int)(splits * n_tiles);
      pl.dyn_lds = 0;
      pl.ws_bytes = splits > 1 ? kCounterBytes + (size_t)n_tiles * splits * pl.bm * kDskCols *
                                                     sizeof(float)
                               : 0;
      return pl;
    }
  }
  // five to sixteen dense rows, k % 128 == 0: one MFMA row tile per 16
  // columns, whole K, every load in flight at once (kind 7, gemv.hip)
  if (!grouped && rows > 4 && rows <= 16 && k % 128 == 0 &&
      env_int("NVFP4_GEMV", 1) != 0) {
    pl.kind = 7;
    pl.bm = 16;
    pl.bn = 16;
    pl.splits = 1;
    pl.k_split = (int)k;
    pl.n_tiles = (int)((n + 15) / 16);
    pl.max_tiles = pl.n_tiles;
    pl.grid = pl.n_tiles;
    pl.dyn_lds = 0;
    pl.ws_bytes = 0;
    return pl;
  }
  const int64_t avg = grouped ? (rows + num_experts - 1) / (num_experts > 0 ? num_experts : 1)
                              : rows;
  int bm = avg <= 16 ? 16 : (avg <= 32 ? 32 : 64);
  if (grouped && avg > 8 && avg <= 24) bm = 32;  // one row tile for most experts
  // dense products up to 128 rows are bound by the load pipeline, not by
  // dequantization: 32-row tiles on 128 columns (two workgroups per CU) fill
  // every resident slot where 64-row tiles on 256 columns leave CUs idle
  // (N = 4096, K = 7168: 19-26 us against 26-30 us for 33-128 rows)
  if (!grouped && rows > 32 && rows <= 128) bm = 32;
  const int force_bm = env_int("NVFP4_BM", 0);
  if (force_bm == 16 || force_bm == 32 || force_bm == 64) bm = force_bm;
  pl.bm = bm;
  choose_kernel(pl, rows, n, k, grouped, cu_count);
  // the large-M kernel keeps no schedule (dense only)
  pl.dyn_lds = pl.kind == 3 ? 0 : sched_lds_bytes(grouped ? num_experts : 1);
  bm = pl.bm;
  pl.n_tiles = (int)((n + pl.bn - 1) / pl.bn);
  // Upper bound on output tiles: each non-empty expert adds at most one
  // partial row tile beyond rows / bm.
  const int64_t mt_bound = grouped ? (rows + bm - 1) / bm + std::min<int64_t>(num_experts, rows)
                                   : (rows + bm - 1) / bm;
  const int64_t max_tiles = mt_bound * pl.n_tiles;
  const int64_t occ = occupancy_for(pl);
  const int64_t slots = (int64_t)cu_count * occ;
  // Split K only when there are too few tiles to occupy the resident slots.
  const int align = pl.fast ? 64 : 16;
  const int kc = pl.fast ? kRingKC : kKC;
  int splits = 1;
  const int64_t tiles_est = grouped ? std::min<int64_t>(num_experts, rows) * pl.n_tiles
                                    : max_tiles;
  if (allow_split && tiles_est < slots) {
    // as many splits as keep every unit in the first round (one more would
    // start a second round of mostly idle slots); each split keeps at least
    // kMinSplitStages K stages: below that the per-unit pipeline fill and the
    // partial-tile hand-off cost more than the extra parallelism buys
    // (measured on the decode shapes)
    int64_t want = slots / tiles_est;
    const int64_t kmax = std::max<int64_t>(1, k / (kMinSplitStages * kc));
    splits = (int)std::min<int64_t>(want, kmax);
  }
  const int force_s = env_int("NVFP4_SPLITK", 0);
  if (force_s > 0 && allow_split) splits = force_s;
  if (max_tiles > kMaxCounters) splits = 1;
  int64_t ksplit = (k + splits - 1) / splits;
  ksplit = (ksplit + align - 1) / align * align;
  splits = (int)((k + ksplit - 1) / ksplit);
  pl.splits = splits;
  pl.k_split = (int)ksplit;
  pl.max_tiles = (int)max_tiles;
  const int64_t units_bound = max_tiles * splits;
  pl.grid = (int)std::max<int64_t>(1, std::min<int64_t>(slots, units_bound));
  // tuning / test override: cap the persistent grid, so that every workgroup
  // walks several units (rounds, cross-unit prefetch) even on small products
  const int force_grid = env_int("NVFP4_GRID", 0);
  if (force_grid > 0) pl.grid = std::min(pl.grid, force_grid);
  pl.ws_bytes = splits > 1
                    ? kCounterBytes + (size_t)max_tiles * splits * bm * pl.bn * sizeof(float)
                    : 0;
  return pl;
}

bool plan_pairs_tiles(const GemmPlan& pl) {
  // K-phase kinds 1 / 2 and the fallback keep two or four tiles per wave;
  // kind 4 (64 columns) keeps one; the large-M kernel is dense only
  return pl.kind == 0 || pl.kind == 1 || pl.kind == 2;
}

// Name of the kernel instantiation launch_gemm runs for a plan (as profilers
// print it), for tooling that reports per-kernel figures.
const char* plan_kernel_name(const GemmPlan& pl, bool gather) {
  if (pl.kind == 6) {
    static const char* kGemv[] = {"nvfp4::gemv_kernel<1>", "nvfp4::gemv_kernel<2>",
                                  "nvfp4::gemv_kernel<3>", "nvfp4::gemv_kernel<4>",
                                  "nvfp4::gemv_kernel<5>", "nvfp4::gemv_kernel<6>"};
    return kGemv[std::min(std::max(pl.bm, 1), kGemvMaxRows) - 1];
  }
  if (pl.kind == 7) {
    // the template argument is the number of 128-deep K groups per wave
    static const char* kDec[] = {"nvfp4::decode_mfma_kernel<1>", "nvfp4::decode_mfma_kernel<2>",
                                 "nvfp4::decode_mfma_kernel<3>", "nvfp4::decode_mfma_kernel<4>",
                                 "nvfp4::decode_mfma_kernel<5>", "nvfp4::decode_mfma_kernel<6>",
                                 "nvfp4::decode_mfma_kernel<7>", "nvfp4::decode_mfma_kernel<8>"};
    const int per_wave = (pl.k_split / 128 + kGemvWaves - 1) / kGemvWaves;
    return kDec[std::min(std::max(per_wave, 1), 8) - 1];
  }
  if (pl.kind == 8) {
    static const char* kDsk[] = {"nvfp4::decode_sk_kernel<1>", "nvfp4::decode_sk_kernel<2>",
                                 "nvfp4::decode_sk_kernel<3>", "nvfp4::decode_sk_kernel<4>"};
    return kDsk[std::min(std::max(pl.bm / 16, 1), 4) - 1];
  }
  if (pl.kind == 3) return "nvfp4::gemm_lm_kernel";
#define NVFP4_KP_NAME(BM, NS, KW, BN) \
  return gather ? "nvfp4::gemm_kp_kernel<" #BM ", " #NS ", " #KW ", " #BN ", true, false>" \
                : "nvfp4::gemm_kp_kernel<" #BM ", " #NS ", " #KW ", " #BN ", false, false>"
  if (pl.kind == 1) {
    if (pl.bm == 16) NVFP4_KP_NAME(16, 5, 4, 128);
    NVFP4_KP_NAME(32, 4, 4, 128);
  }
  if (pl.kind == 4) NVFP4_KP_NAME(16, 5, 4, 64);
  if (pl.kind == 2) {
    if (pl.bm == 16) NVFP4_KP_NAME(16, 5, 8, 256);
    if (pl.bm == 32) NVFP4_KP_NAME(32, 5, 8, 256);
    NVFP4_KP_NAME(64, 4, 8, 256);
  }
#undef NVFP4_KP_NAME
  if (pl.bm == 16) return "nvfp4::gemm_reg_kernel<16>";
  if (pl.bm == 32) return "nvfp4::gemm_reg_kernel<32>";
  return "nvfp4::gemm_reg_kernel<64>";
}

hipError_t launch_gemm(const GemmPlan& pl, const GemmParams& p, hipStream_t stream) {
  if (pl.kind == 6 || pl.kind == 7 || pl.kind == 8) return launch_gemv(pl, p, stream);
  dim3 grid(pl.grid);
#define NVFP4_KP(BM, NS, KW, BN)                                                           \
  do {                                                                                     \
    if (p.row_index != nullptr)                                                            \
      hipLaunchKernelGGL((gemm_kp_kernel<BM, NS, KW, BN, true>), grid, dim3(KW * 64),      \
                         pl.dyn_lds, stream, p);                                           \
    else                                                                                   \
      hipLaunchKernelGGL((gemm_kp_kernel<BM, NS, KW, BN>), grid, dim3(KW * 64), pl.dyn_lds, \
                         stream, p);                                                       \
  } while (0)
  if (pl.kind == 3) {
    hipLaunchKernelGGL(gemm_lm_kernel, grid, dim3(LmLayout::kWaves * 64), 0, stream, p);
  } else if (pl.kind == 1) {
    if (pl.bm == 16) NVFP4_KP(16, 5, 4, 128);
    else NVFP4_KP(32, 4, 4, 128);
  } else if (pl.kind == 4) {
    NVFP4_KP(16, 5, 4, 64);
  } else if (pl.kind == 2) {
    if (pl.bm == 16) NVFP4_KP(16, 5, 8, 256);
    else if (pl.bm == 32) NVFP4_KP(32, 5, 8, 256);
    else NVFP4_KP(64, 4, 8, 256);
  } else {
    dim3 block(kRegThreads);
    if (pl.bm == 16) hipLaunchKernelGGL(gemm_reg_kernel<16>, grid, block, pl.dyn_lds, stream, p);
    else if (pl.bm == 32)
      hipLaunchKernelGGL(gemm_reg_kernel<32>, grid, block, pl.dyn_lds, stream, p);
    else hipLaunchKernelGGL(gemm_reg_kernel<64>, grid, block, pl.dyn_lds, stream, p);
  }
#undef NVFP4_KP
  return hipGetLastError();
}

bool plan_fusable(const GemmPlan& up, const GemmPlan& down) {
  return (up.kind == 1 || up.kind == 2) && up.kind == down.kind && up.bm == down.bm &&
         up.bn == down.bn && up.nslot == down.nslot && up.splits == 1 && down.splits == 1 &&
         up.fast && down.fast;
}

// Resident workgroups per CU of the fused instantiation of a plan's kernel.
int fused_occupancy(const GemmPlan& pl) {
  const int dyn = pl.dyn_lds;
  if (pl.kind == 1)
    return pl.bm == 16 ? occupancy_of(gemm_kp_kernel<16, 5, 4, 128, false, true>, 256, dyn)
                       : occupancy_of(gemm_kp_kernel<32, 4, 4, 128, false, true>, 256, dyn);
  return pl.bm == 16 ? occupancy_of(gemm_kp_kernel<16, 5, 8, 256, false, true>, 512, dyn)
         : pl.bm == 32 ? occupancy_of(gemm_kp_kernel<32, 5, 8, 256, false, true>, 512, dyn)
                       : occupancy_of(gemm_kp_kernel<64, 4, 8, 256, false, true>, 512, dyn);
}

const char* fused_kernel_name(const GemmPlan& pl) {
  if (pl.kind == 1)
    return pl.bm == 16 ? "nvfp4::gemm_kp_kernel<16, 5, 4, 128, false, true>"
                       : "nvfp4::gemm_kp_kernel<32, 4, 4, 128, false, true>";
  return pl.bm == 16 ? "nvfp4::gemm_kp_kernel<16, 5, 8, 256, false, true>"
         : pl.bm == 32 ? "nvfp4::gemm_kp_kernel<32, 5, 8, 256, false, true>"
                       : "nvfp4::gemm_kp_kernel<64, 4, 8, 256, false, true>";
}

hipError_t launch_gemm_fused(const GemmPlan& pl, int grid, const GemmParams& p,
                             hipStream_t stream) {
  const dim3 g((unsigned)grid);
#define NVFP4_KPF(BM, NS, KW, BN) \
  hipLaunchKernelGGL((gemm_kp_kernel<BM, NS, KW, BN, false, true>), g, dim3(KW * 64), pl.dyn_lds, \
                     stream, p)
  if (pl.kind == 1) {
    if (pl.bm == 16) NVFP4_KPF(16, 5, 4, 128);
    else NVFP4_KPF(32, 4, 4, 128);
  } else if (pl.kind == 2) {
    if (pl.bm == 16) NVFP4_KPF(16, 5, 8, 256);
    else if (pl.bm == 32) NVFP4_KPF(32, 5, 8, 256);
    else NVFP4_KPF(64, 4, 8, 256);
  } else {
    return hipErrorInvalidValue;
  }
#undef NVFP4_KPF
  return hipGetLastError();
}

}  // namespace nvfp4
