// inst_tile.hip -- kernel instances for one (input type, output type,
// trans_a, trans_b) combination, selected at compile time by
//   TG_IN, TG_OUT (element types), TG_TA, TG_TB (0/1) and
//   TG_TABLE_TILE, TG_TABLE_GENERIC (names of the exported tables).
// The library compiles this file once per combination.
#include "tiles.hpp"
#include "tile_gemm.hpp"
#include "generic_gemm.hpp"


namespace tg {
namespace {

template <int T>
constexpr KernelFn tile_k() {
  constexpr TileShape s = kTiles[T];
  return &tile_gemm_kernel<TG_IN, TG_OUT, s.bm, s.bn, s.bk, s.wm, s.wn, s.stages, s.occ,
                           s.dw ? s.dw : s.wm * s.wn, TG_TA != 0, TG_TB != 0>;
}
template <int T>
constexpr KernelFn generic_k() {
  constexpr TileShape s = kGenericTiles[T];
  return &generic_gemm_kernel<TG_IN, TG_OUT, s.bm, s.bn, s.bk, s.wm, s.wn, TG_TA != 0, TG_TB != 0>;
}

}  // namespace

extern const KernelFn TG_TABLE_TILE[kNumTiles];
extern const KernelFn TG_TABLE_GENERIC[kNumGeneric];

#define TG_TILE_ENTRY(i) tile_k<i>()
const KernelFn TG_TABLE_TILE[kNumTiles] = {TG_TILE_ENTRY(0), TG_TILE_ENTRY(1), TG_TILE_ENTRY(2), TG_TILE_ENTRY(3),
                                          TG_TILE_ENTRY(4), TG_TILE_ENTRY(5), TG_TILE_ENTRY(6), TG_TILE_ENTRY(7),
                                          TG_TILE_ENTRY(8), TG_TILE_ENTRY(9), TG_TILE_ENTRY(10), TG_TILE_ENTRY(11),
                                          TG_TILE_ENTRY(12), TG_TILE_ENTRY(13), TG_TILE_ENTRY(14), TG_TILE_ENTRY(15)};
const KernelFn TG_TABLE_GENERIC[kNumGeneric] = {generic_k<0>(), generic_k<1>()};
static_assert(kNumTiles == 16 && kNumGeneric == 2, "update the instance tables");

}  // namespace tg
