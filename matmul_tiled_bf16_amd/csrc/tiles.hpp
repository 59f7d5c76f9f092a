// tiles.hpp -- tile tables shared by the planner and the kernel instances.
//
// Each entry fixes the work-group tile (BM x BN), the K step (BK), the wave
// grid (WM x WN, 64 lanes per wave) and the LDS ring depth.  The LDS budget
// stages * (BM*BK + BK*BN) * 2 bytes stays within the 160 KiB one gfx950
// work-group may hold ("Optimize Triton Block Parameters", Step 2: stages
// times the A/B tile pair, checked against on-chip capacity).
#pragma once

namespace tg {

// Kernel behind a tile entry.
enum TileKind {
  kTileKernel = 0,  // tile_gemm_kernel (tile_gemm.hpp)
  kPingPong = 1,    // pingpong_gemm_kernel without epilogue: persistent when there is enough work
  kPingPongEpi = 2,  // pingpong_gemm_kernel with the alpha/beta/bias epilogue (one tile per work-group)
  kPanel = 3         // panel_gemm_kernel: short K, A resident in registers along a row panel of C
};

struct TileShape {
  int bm, bn, bk, wm, wn, stages;
  int occ = 1;  // work-groups meant to share one CU (register/LDS budget per wave follows)
  int dw = 0;   // waves that issue the HBM->LDS copies (0: all of them)
  int kind = kTileKernel;
};

constexpr TileShape kTiles[] = {
    {64, 64, 64, 2, 2, 2},     // 0: 32x32 per wave -- small and ragged problems
    {128, 128, 64, 2, 2, 2},   // 1: 64x64 per wave
    {256, 256, 32, 2, 2, 4},   // 2: 128x128 per wave, 4-deep ring -- large, compute-bound
    {256, 128, 64, 2, 2, 2},   // 3: 128x64 per wave
    {128, 256, 64, 2, 2, 2},   // 4: 64x128 per wave
    {32, 128, 64, 1, 4, 2},    // 5: one 32-row tile -- thin M
    {128, 128, 32, 2, 2, 4},   // 6: 64x64 per wave, 4-deep ring
    {256, 256, 64, 2, 2, 2},   // 7: 128x128 per wave, 2-deep ring
    {256, 256, 32, 2, 4, 4},   // 8: 8 waves (2 per SIMD), 128x64 per wave, 4-deep ring
    {256, 256, 64, 2, 4, 2},   // 9: 8 waves, 128x64 per wave, 2-deep ring
    // two work-groups per CU (<= 80 KiB LDS, <= 256 registers per lane each)
    {256, 128, 32, 2, 2, 3, 2},  // 10: 128x64 per wave, 3-deep ring
    {128, 256, 32, 2, 2, 3, 2},  // 11: 64x128 per wave, 3-deep ring
    {256, 128, 32, 2, 2, 2, 2},  // 12: 128x64 per wave, 2-deep ring
    {128, 128, 64, 2, 2, 2, 2},  // 13: 64x64 per wave
    // 8 waves, copies issued by the second wave of each SIMD only
    {256, 256, 64, 2, 4, 2, 1, 4},  // 14
    {256, 256, 32, 2, 4, 4, 1, 4},  // 15
    // three or four work-groups per CU: small rings for short K, where the
    // loads are latency-bound and only concurrency hides them
    {128, 128, 32, 2, 2, 2, 4},  // 16: 32 KiB
    {128, 128, 32, 2, 2, 3, 3},  // 17: 48 KiB
    {64, 128, 64, 2, 2, 2, 3},   // 18: 32x64 per wave, 48 KiB
    {128, 64, 64, 2, 2, 2, 4},   // 19: 64x32 per wave, 32 KiB
    // 5-deep rings (160 KiB): three K steps between a stage's copies and
    // their use -- a single wave per SIMD has nothing else to hide latency
    {256, 256, 32, 2, 2, 5},     // 20: 4 waves, 128x128 per wave
    {256, 256, 32, 2, 4, 5},     // 21: 8 waves, 128x64 per wave
    // 8 waves, 4 of them copy: persistent work-groups whose copy waves
    // prefetch while the other waves store (split mode)
    {128, 128, 64, 2, 4, 2, 2, 4},  // 22: 64x32 per wave, 64 KiB
    // 8 waves in two groups that alternate MFMA and memory phases
    // (pingpong_gemm.hpp): 128x64 per wave, 64-deep K steps, three A and two
    // B LDS buffers (160 KiB); the second entry adds the epilogue
    {256, 256, 64, 2, 4, 2, 1, 4, kPingPong},     // 23
    {256, 256, 64, 2, 4, 2, 1, 4, kPingPongEpi},  // 24
    // 4 waves walking runs of 128 x 128 tiles along a row panel of C, K <=
    // 128 (panel_gemm.hpp): A in registers, two B LDS buffers (64 KiB), two
    // work-groups per CU
    {128, 128, 128, 2, 2, 2, 2, 0, kPanel},  // 25
    // 64x64 tiles with deep rings for small, latency-bound products: with
    // a K step's MFMAs far shorter than a copy's round trip, the time per
    // step is the round trip divided by the steps in flight
    {64, 64, 64, 2, 2, 4, 2},  // 26: 4-deep ring, 64 KiB
    {64, 64, 32, 2, 2, 5, 3},  // 27: 5-deep ring of 32-deep steps, 40 KiB
};
constexpr int kPingPongTile = 23, kPingPongEpiTile = 24, kPanelTile = 25;
constexpr int kPanelKMax = kTiles[kPanelTile].bk;  // the panel kernel holds all of K at once
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Tiles a grouped launch may take (indices into kTiles): small and ragged
// groups, two HBM/MFMA-balanced 128x128 shapes, the large 8-wave tile, and
// three shapes with three or four work-groups per CU for groups that stream
// their B operands (more copies in flight per CU).
constexpr int kGroupTiles[] = {0, 13, 1, 8, 17, 16, 19};
constexpr int kNumGroup = sizeof(kGroupTiles) / sizeof(kGroupTiles[0]);

constexpr TileShape kGenericTiles[] = {
    {64, 64, 64, 2, 2, 2},
    {128, 128, 64, 2, 2, 2},
};
constexpr int kNumGeneric = sizeof(kGenericTiles) / sizeof(kGenericTiles[0]);

constexpr int lds_bytes_of(const TileShape& t) {
  return t.kind == kPanel ? t.stages * t.bk * t.bn * 2
         : t.kind != kTileKernel ? (3 * t.bm * t.bk + 2 * t.bk * t.bn) * 2
                                 : t.stages * (t.bm * t.bk + t.bk * t.bn) * 2;
}

// Whether the tile kernel can run persistently: the first wait of a
// prefetched item counts the copy instructions of the stages after the first
// one plus the item's store instructions, and that count must fit the 6-bit
// vector-memory counter.
// Whether the tile kernel can run in split mode for a given output element
// size: dedicated copy waves, a C tile that fits the ring's LDS in one band,
// and a band that divides evenly over the waves that store it.
constexpr bool split_ok(const TileShape& t, int out_size) {
  if (t.kind != kTileKernel) return false;
  const int nw = t.wm * t.wn;
  const int stores = nw - (t.dw ? t.dw : nw);
  const int c_bytes = t.bm * t.bn * out_size;
  return stores > 0 && t.bn * out_size / 16 >= 4 && c_bytes <= lds_bytes_of(t) &&
         (c_bytes / 16) % (stores * 64) == 0;
}

constexpr bool persist_ok(const TileShape& t) {
  if (t.kind != kTileKernel) return false;
  const int copy_waves = t.dw ? t.dw : t.wm * t.wn;
  const int per_step = (t.bm * t.bk * 2 / 1024) / copy_waves + (t.bk * t.bn * 2 / 1024) / copy_waves;
  const int d = t.stages >= 3 ? t.stages - 1 : t.stages;
  const int stores = (t.bm / t.wm / 32) * (t.bn / t.wn / 32) * 4;
  return (d - 1) * per_step + stores < 64;
}

// Skinny (M <= 32) streaming kernel: MB 16-row blocks of A and C, NB 16-row
// blocks of B (16*NB columns of C) per work-group, WAVES waves, STAGES LDS
// stage buffers of SK k-elements.  LDS is static: STAGES * (16*NB + 16*MB)
// rows * 2*SK bytes.
struct SkinnyShape {
  int mb, nb, waves, stages, sk;
};
constexpr SkinnyShape kSkinny[] = {
    {1, 1, 4, 3, 256},  // 0: M <= 16, 16 columns, 48 KiB (three work-groups per CU)
    {2, 2, 8, 4, 256},  // 1: M <= 32, 128 KiB
    {1, 1, 2, 4, 256},  // 2: M <= 16, 16 columns, 2 waves, 64 KiB
    {1, 1, 8, 4, 256},  // 3: M <= 16, 16 columns, 8 waves, 64 KiB
    {1, 1, 4, 5, 256},  // 4: M <= 16, 16 columns, 80 KiB (two work-groups per CU)
    {1, 1, 4, 4, 256},  // 5: M <= 16, 16 columns, 64 KiB
    {2, 1, 4, 3, 256},  // 6: M <= 32, 16 columns, 72 KiB
    {1, 2, 8, 4, 256},  // 7: M <= 16, 32 columns, 96 KiB
};
constexpr int kNumSkinny = sizeof(kSkinny) / sizeof(kSkinny[0]);
constexpr int skinny_lds_of(const SkinnyShape& s) { return s.stages * (16 * s.nb + 16 * s.mb) * 2 * s.sk; }

}  // namespace tg
