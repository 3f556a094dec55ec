// kp_layout.hpp -- LDS layout and per-stage load counts of the K-phase GEMM
// kernel (gemm.hip), as plain constant expressions so that host code (the
// schedule model in the tests) sees exactly the numbers the kernel uses.
//
// A work unit is (expert, row tile of BM rows, column tile of BN weight rows,
// K split); K advances in kRingKC-deep stages held in an NSLOT-deep LDS ring
// (packed weights BN x 64 B, then activations BM x 256 B), block scales in
// windows of kWinStages stages in three buffers after the ring.  KW waves
// split a stage as wave w = 2 ch + kp: columns [CPW ch, CPW ch + CPW), K half
// kp.  Every load is a 1 KB buffer_load ... lds (64 lanes x 16 B).
#pragma once

namespace nvfp4 {

constexpr int kRingKC = 128;  // K per stage

template <int BM, int NSLOT, int KW, int BN>
struct KpLayout {
  static constexpr int kCPW = 2 * BN / KW;          // columns per wave
  static constexpr int kNJ = kCPW / 16;             // MFMA column tiles per wave
  static constexpr int kW = 0;                      // BN rows x 64 B packed nibbles
  static constexpr int kX = BN * 64;                // BM rows x 256 B activations
  static constexpr int kStage = kX + BM * 256;
  static constexpr int kWPerWave = BN / 16 / KW;    // 1 KB (16-row) weight loads per wave
  static constexpr int kXInstr = BM / 4;            // 1 KB (4-row) activation loads
  static constexpr int kXPerWave = kXInstr >= KW ? kXInstr / KW : 1;
  static constexpr int kLoadsPerStage = kWPerWave + kXPerWave;
  // A scale window covers kWinStages stages (8 bytes per row each) of one
  // unit and goes out just before its first stage.  Windows take three
  // buffers in stream order; a buffer is refilled three windows later, after
  // every wave has read the window it held (NSLOT <= kWinStages + 1 keeps
  // that true even across units whose last window is short).
  static constexpr int kWinStages = NSLOT <= 3 ? 2 : 4;
  static constexpr int kWinBufs = 3;
  static constexpr int kWinRow = 8 * kWinStages;    // window bytes per weight row
  static constexpr int kWinBytes = BN * kWinRow;
  static constexpr int kSInstr = kWinBytes / 1024;  // 1 KB scale window loads
  static constexpr int kSWin = NSLOT * kStage;
  static constexpr int kTotal = kSWin + kWinBufs * kWinBytes;
  static constexpr int kSPerWave = kSInstr >= KW ? kSInstr / KW : 1;
  // K-half exchange at the end of a unit: 1 KB chunks, kRedSlots ring slots
  static constexpr int kChunksPerStage = kStage / 1024;
  static constexpr int kRedChunks = KW * (BM / 16) * (kNJ / 2);
  static constexpr int kRedSlots = (kRedChunks + kChunksPerStage - 1) / kChunksPerStage;
  // stages of the next unit issued during a unit's last iterations (the
  // other ring slots hold the exchange)
  static constexpr int kPrefetch = NSLOT - kRedSlots;
  // vector memory instructions of a unit's epilogue when the next unit's
  // first stages are prefetched: 16-byte stores of the output tile, as many
  // as the widest output (BM x BN FP32 values) takes per wave
  static constexpr int kEpiStores = (BM * BN * 4 + 16 * KW * 64 - 1) / (16 * KW * 64);
  static_assert(kWPerWave >= 1 && kSInstr >= 1 && (kSInstr < KW || kSInstr % KW == 0),
                "load split");
  static_assert(NSLOT <= kWinStages + 1, "window buffers are reused in time");
  static_assert(kNJ % 2 == 0, "column tiles split between the K halves");
  static_assert(NSLOT >= 3 && NSLOT <= 5, "windows are issued one window ahead");
  static_assert(kStage % 1024 == 0 && kRedSlots < NSLOT, "exchange fits the ring");
  static_assert(kPrefetch >= 1 && kPrefetch <= kWinStages, "prefetch within window 0");
};

// The configurations gemm.hip instantiates: <BM, NSLOT, KW, BN>.
constexpr int kKpConfigs[][4] = {{16, 5, 4, 128}, {32, 4, 4, 128}, {16, 5, 4, 64},
                                 {16, 5, 8, 256}, {32, 5, 8, 256}, {64, 4, 8, 256}};

}  // namespace nvfp4
