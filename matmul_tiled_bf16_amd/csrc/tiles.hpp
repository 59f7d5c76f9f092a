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
  kPanel = 3,        // panel_gemm_kernel: short K, A resident in registers along a row panel of C
  kKSlice = 4,       // kslice_gemm_kernel: 64x64 tiles whose four waves split K (short chains)
  kTileEpi = 5       // tile_gemm_kernel with the alpha/beta/bias epilogue compiled in
};

struct TileShape {
  int bm, bn, bk, wm, wn, stages;
  int occ = 1;  // work-groups meant to share one CU (register/LDS budget per wave follows)
  int dw = 0;   // waves that issue the HBM->LDS copies (0: all of them)
  int kind = kTileKernel;
};

// Only the shapes the planner and the grouped launch choose are built.
constexpr TileShape kTiles[] = {
    {64, 64, 64, 2, 2, 2},     // 0: 32x32 per wave -- small and ragged problems, short K
    {128, 128, 64, 2, 2, 2},   // 1: 64x64 per wave -- MFMA-bound products with 128-256 such tiles
    {32, 128, 64, 1, 4, 2},    // 2: one 32-row tile -- thin M that the skinny kernel does not take
    {256, 256, 32, 2, 4, 4},   // 3: 8 waves (2 per SIMD), 128x64 per wave, 4-deep ring -- grouped
                               //    MFMA-bound launches; K = 0 on a ping-pong plan
    {128, 128, 64, 2, 2, 2, 2},  // 4: 64x64 per wave, two work-groups per CU -- HBM-bound products
    // three or four work-groups per CU: small rings for short K, where the
    // loads are latency-bound and only concurrency hides them (grouped launches)
    {128, 128, 32, 2, 2, 2, 4},  // 5: 32 KiB
    {128, 128, 32, 2, 2, 3, 3},  // 6: 48 KiB
    {128, 64, 64, 2, 2, 2, 4},   // 7: 64x32 per wave, 32 KiB
    // 8 waves in two groups that alternate MFMA and memory phases
    // (pingpong_gemm.hpp): 128x64 per wave, 64-deep K steps, three A and two
    // B LDS buffers (160 KiB); the second entry adds the epilogue
    {256, 256, 64, 2, 4, 2, 1, 4, kPingPong},     // 8
    {256, 256, 64, 2, 4, 2, 1, 4, kPingPongEpi},  // 9
    // 4 waves walking runs of 128 x 128 tiles along a row panel of C, K <=
    // 128 (panel_gemm.hpp): A in registers, two B LDS buffers (64 KiB), two
    // work-groups per CU
    {128, 128, 128, 2, 2, 2, 2, 0, kPanel},  // 10
    // 64x64 tiles with a deep ring for small, latency-bound products with a
    // long K: with a K step's MFMAs far shorter than a copy's round trip, the
    // time per step is the round trip divided by the steps in flight
    {64, 64, 64, 2, 2, 4, 2},  // 11: 4-deep ring, 64 KiB
    // 64x64 tiles whose four waves each walk a quarter of K through a ring
    // of their own (kslice_gemm.hpp): 32-deep steps, four stages per wave
    // (a fifth measured slower: 1000^3 10.4 -> 11.0 us)
    {64, 64, 32, 2, 2, 4, 1, 0, kKSlice},  // 12: 4 x 32 KiB
    // the tile kernel with the epilogue compiled in: the launcher sends a call
    // with an epilogue planned on a tile-kernel entry to the twin of its
    // shape class (the other entries leave the epilogue's registers free)
    {64, 64, 64, 2, 2, 2, 1, 0, kTileEpi},      // 13: twin of 0, 2, 11
    {128, 128, 64, 2, 2, 2, 1, 0, kTileEpi},    // 14: twin of 1, 5, 6, 7
    {256, 256, 32, 2, 4, 4, 1, 0, kTileEpi},    // 15: twin of 3
    {128, 128, 64, 2, 2, 2, 2, 0, kTileEpi},    // 16: twin of 4 and 17
    // 256x128, 8 waves of 64x64 each, one work-group per CU (96 KiB): HBM-bound
    // products with N <= 256, whose B panels 128-row tiles read twice as often
    {256, 128, 64, 4, 2, 2, 1},  // 17
};
constexpr int kSmallTile = 0, kMfmaMidTile = 1, kThinTile = 2, kWideTile = 3, kHbmTile = 4, kDeepSmallTile = 11;
constexpr int kKSliceTile = 12, kTallTile = 17;
// the epilogue twin of a tile-kernel entry
constexpr int epi_twin(int t) {
  return t == 3 ? 15 : (t == 4 || t == 17) ? 16 : (t == 1 || t == 5 || t == 6 || t == 7) ? 14 : 13;
}
constexpr int kPingPongTile = 8, kPingPongEpiTile = 9, kPanelTile = 10;
constexpr int kPanelKMax = kTiles[kPanelTile].bk;  // the panel kernel holds all of K at once
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Tiles a grouped launch may take (indices into kTiles): small and ragged
// groups, two HBM/MFMA-balanced 128x128 shapes, the large 8-wave tile, and
// three shapes with three or four work-groups per CU for groups that stream
// their B operands (more copies in flight per CU).
constexpr int kGroupTiles[] = {kSmallTile, kHbmTile, kMfmaMidTile, kWideTile, 6, 5, 7};
constexpr int kNumGroup = sizeof(kGroupTiles) / sizeof(kGroupTiles[0]);

constexpr TileShape kGenericTiles[] = {
    {64, 64, 64, 2, 2, 2},
    {128, 128, 64, 2, 2, 2},
};
constexpr int kNumGeneric = sizeof(kGenericTiles) / sizeof(kGenericTiles[0]);

constexpr int lds_bytes_of(const TileShape& t) {
  return t.kind == kPanel    ? t.stages * t.bk * t.bn * 2
         : t.kind == kKSlice ? t.wm * t.wn * t.stages * (t.bm * t.bk + t.bk * t.bn) * 2
         : (t.kind == kPingPong || t.kind == kPingPongEpi) ? (3 * t.bm * t.bk + 2 * t.bk * t.bn) * 2
                                                           : t.stages * (t.bm * t.bk + t.bk * t.bn) * 2;
}

// Whether the tile kernel can run persistently: the first wait of a
// prefetched item counts the copy instructions of the stages after the first
// one plus the item's store instructions, and that count must fit the 6-bit
// vector-memory counter.
constexpr bool persist_ok(const TileShape& t) {
  if (t.kind != kTileKernel && t.kind != kTileEpi) return false;
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
};
constexpr int kNumSkinny = sizeof(kSkinny) / sizeof(kSkinny[0]);
constexpr int skinny_lds_of(const SkinnyShape& s) { return s.stages * (16 * s.nb + 16 * s.mb) * 2 * s.sk; }

}  // namespace tg
