// Prints the K-phase kernel's layout constants (kp_layout.hpp, the header the
// kernel itself includes) for every instantiated configuration, one line
// each, for the host model of the kernel's schedule (test_kp_schedule_model).
#include <cstdio>

#include "../../block_scaled_fp4_nibble_amd/csrc/kp_layout.hpp"

template <int BM, int NSLOT, int KW, int BN>
void dump() {
  using L = nvfp4::KpLayout<BM, NSLOT, KW, BN>;
  std::printf(
      "BM=%d NSLOT=%d KW=%d BN=%d kNJ=%d kW=%d kX=%d kStage=%d kWPerWave=%d kXInstr=%d "
      "kXPerWave=%d kLoadsPerStage=%d kWinStages=%d kWinBufs=%d kWinBytes=%d kSInstr=%d "
      "kSWin=%d kTotal=%d kSPerWave=%d kChunksPerStage=%d kRedChunks=%d kRedSlots=%d "
      "kPrefetch=%d kEpiStores=%d RingKC=%d\n",
      BM, NSLOT, KW, BN, L::kNJ, L::kW, L::kX, L::kStage, L::kWPerWave, L::kXInstr,
      L::kXPerWave, L::kLoadsPerStage, L::kWinStages, L::kWinBufs, L::kWinBytes, L::kSInstr,
      L::kSWin, L::kTotal, L::kSPerWave, L::kChunksPerStage, L::kRedChunks, L::kRedSlots,
      L::kPrefetch, L::kEpiStores, nvfp4::kRingKC);
}

int main() {
  static_assert(sizeof(nvfp4::kKpConfigs) / sizeof(nvfp4::kKpConfigs[0]) == 6, "config list");
  dump<16, 5, 4, 128>();
  dump<32, 4, 4, 128>();
  dump<16, 5, 4, 64>();
  dump<16, 5, 8, 256>();
  dump<32, 5, 8, 256>();
  dump<64, 4, 8, 256>();
  return 0;
}
