// inst_tile.hip -- kernel instances for one (input type, output type,
// trans_a, trans_b) combination, selected at compile time by
//   TG_IN, TG_OUT (element types), TG_TA, TG_TB (0/1) and
//   TG_TABLE_TILE, TG_TABLE_GENERIC, TG_TABLE_GROUP (names of the exported tables).
// The library compiles this file once per combination.
#include <array>
#include <utility>

#include "tiles.hpp"
#include "tile_gemm.hpp"
#include "pingpong_gemm.hpp"
#include "panel_gemm.hpp"
#include "kslice_gemm.hpp"
#include "generic_gemm.hpp"


namespace tg {
namespace {

template <int T>
constexpr KernelFn tile_k() {
  constexpr TileShape s = kTiles[T];
  if constexpr (s.kind == kPingPong)
    return &pingpong_gemm_kernel<TG_IN, TG_OUT, TG_TA != 0, TG_TB != 0, false>;
  else if constexpr (s.kind == kPingPongEpi)
    return &pingpong_gemm_kernel<TG_IN, TG_OUT, TG_TA != 0, TG_TB != 0, true>;
  else if constexpr (s.kind == kPanel && TG_TA == 0)
    return &panel_gemm_kernel<TG_IN, TG_OUT, TG_TB != 0>;
  else if constexpr (s.kind == kPanel)
    return nullptr;  // A stored K x M: the launcher sends these to a tile kernel
  else if constexpr (s.kind == kKSlice)
    return &kslice_gemm_kernel<TG_IN, TG_OUT, TG_TA != 0, TG_TB != 0, s.stages>;
  else
    return &tile_gemm_kernel<TG_IN, TG_OUT, s.bm, s.bn, s.bk, s.wm, s.wn, s.stages, s.occ,
                             s.dw ? s.dw : s.wm * s.wn, TG_TA != 0, TG_TB != 0, s.kind == kTileEpi>;
}
template <int T>
constexpr KernelFn generic_k() {
  constexpr TileShape s = kGenericTiles[T];
  return &generic_gemm_kernel<TG_IN, TG_OUT, s.bm, s.bn, s.bk, s.wm, s.wn, TG_TA != 0, TG_TB != 0>;
}

template <int G>
constexpr GroupFn group_k() {
  constexpr TileShape s = kTiles[kGroupTiles[G]];
  return &group_gemm_kernel<TG_IN, TG_OUT, s.bm, s.bn, s.bk, s.wm, s.wn, s.stages, s.occ,
                            s.dw ? s.dw : s.wm * s.wn, TG_TA != 0, TG_TB != 0>;
}

template <std::size_t... I>
constexpr std::array<GroupFn, sizeof...(I)> group_array(std::index_sequence<I...>) {
  return {group_k<I>()...};
}
template <std::size_t... I>
constexpr std::array<KernelFn, sizeof...(I)> tile_array(std::index_sequence<I...>) {
  return {tile_k<I>()...};
}
template <std::size_t... I>
constexpr std::array<KernelFn, sizeof...(I)> generic_array(std::index_sequence<I...>) {
  return {generic_k<I>()...};
}

}  // namespace

extern const std::array<KernelFn, kNumTiles> TG_TABLE_TILE;
extern const std::array<KernelFn, kNumGeneric> TG_TABLE_GENERIC;
extern const std::array<GroupFn, kNumGroup> TG_TABLE_GROUP;
const std::array<KernelFn, kNumTiles> TG_TABLE_TILE = tile_array(std::make_index_sequence<kNumTiles>{});
const std::array<KernelFn, kNumGeneric> TG_TABLE_GENERIC = generic_array(std::make_index_sequence<kNumGeneric>{});
const std::array<GroupFn, kNumGroup> TG_TABLE_GROUP = group_array(std::make_index_sequence<kNumGroup>{});

}  // namespace tg
