// tgemm.hip -- planner, kernel tables and the C ABI declared in include/tgemm.h.
//
// Planning follows the pages' block-parameter reasoning, restated for CDNA4
// ("Optimize Triton Block Parameters", Steps 1-4 and Performance
// requirements): classify the shape, keep the LDS budget
// stages*(BM*BK + BK*BN)*2 bytes within the 160 KiB a gfx950 work-group may
// hold, give small and ragged problems small tiles so the grid still covers
// the 256 CUs, and take the 16-byte vector loader only where alignment allows
// it ("Triton Optimization Reference", section 6).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <atomic>

#include "../../include/tgemm.h"
#include "common.hpp"
#include "tiles.hpp"

namespace tg {
// Instance tables, one per (input, output, trans_a, trans_b); defined by the
// objects built from inst_tile.hip and inst_skinny.hip.
#define TG_DECLARE(in, out, ta, tb)                                                \
  extern const std::array<KernelFn, kNumTiles> tile_##in##_##out##_##ta##tb;       \
  extern const std::array<KernelFn, kNumGeneric> generic_##in##_##out##_##ta##tb;  \
  extern const std::array<GroupFn, kNumGroup> group_##in##_##out##_##ta##tb;
#define TG_DECLARE_IO(in, out) \
  TG_DECLARE(in, out, 0, 0) TG_DECLARE(in, out, 0, 1) TG_DECLARE(in, out, 1, 0) TG_DECLARE(in, out, 1, 1)
TG_DECLARE_IO(bf16, f32)
TG_DECLARE_IO(bf16, bf16)
TG_DECLARE_IO(f16, f32)
TG_DECLARE_IO(f16, f16)
extern const std::array<KernelFn, kNumSkinny> skinny_table[2][2];
}  // namespace tg

namespace {

using tg::KernelFn;
using tg::kGenericTiles;
using tg::kGroupTiles;
using tg::kNumGeneric;
using tg::kNumGroup;
using tg::kNumSkinny;
using tg::kNumTiles;
using tg::kSkinny;
using tg::kTiles;
using tg::TileShape;

#define TG_ROW(in, out)                                                                           \
  {tg::tile_##in##_##out##_00.data(), tg::tile_##in##_##out##_01.data(), tg::tile_##in##_##out##_10.data(), \
   tg::tile_##in##_##out##_11.data()}
#define TG_GROW(in, out)                                                                                      \
  {tg::generic_##in##_##out##_00.data(), tg::generic_##in##_##out##_01.data(),                              \
   tg::generic_##in##_##out##_10.data(), tg::generic_##in##_##out##_11.data()}

// [in bf16/fp16][out fp32/same][2*trans_a + trans_b]
const KernelFn* const kTileTables[2][2][4] = {{TG_ROW(bf16, f32), TG_ROW(bf16, bf16)},
                                              {TG_ROW(f16, f32), TG_ROW(f16, f16)}};
const KernelFn* const kGenericTables[2][2][4] = {{TG_GROW(bf16, f32), TG_GROW(bf16, bf16)},
                                                 {TG_GROW(f16, f32), TG_GROW(f16, f16)}};
#define TG_GRPROW(in, out)                                                                                \
  {tg::group_##in##_##out##_00.data(), tg::group_##in##_##out##_01.data(), tg::group_##in##_##out##_10.data(), \
   tg::group_##in##_##out##_11.data()}
const tg::GroupFn* const kGroupTables[2][2][4] = {{TG_GRPROW(bf16, f32), TG_GRPROW(bf16, bf16)},
                                                  {TG_GRPROW(f16, f32), TG_GRPROW(f16, f16)}};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The vector kernel reads 16-byte units along each operand's contiguous
// dimension: every leading dimension and contiguous extent must be a multiple
// of 8 elements, and one tile's span of rows must stay addressable by the
// 31-bit buffer offsets.
bool vec_ok(const gemm_plan_t& p) {
  const int64_t a_contig = p.trans_a ? p.m : p.k;
  const int64_t b_contig = p.trans_b ? p.k : p.n;
  const int64_t span = (int64_t)1 << 30;  // 256 rows * ld * 2 bytes < 2^31
  return p.lda % 8 == 0 && p.ldb % 8 == 0 && p.ldc % 8 == 0 && a_contig % 8 == 0 && b_contig % 8 == 0 &&
         a_contig >= 8 && b_contig >= 8 && p.lda * 256 < span && p.ldb * 256 < span && p.ldc * 512 < span;
}

// The skinny kernel reads 16-byte chunks of A's and B's rows along K through
// buffer descriptors whose 31-bit byte offsets span one work-group's rows of
// B (at most 64) or all of A (at most 32 rows), plus the K extent.
bool skinny_ok(const gemm_plan_t& p) {
  const int64_t lim = (int64_t)1 << 31;
  return !p.trans_a && p.trans_b && p.m >= 1 && p.m <= 32 && p.lda % 8 == 0 && p.ldb % 8 == 0 && p.k % 8 == 0 &&
         p.k >= 8 && 2 * (64 * p.ldb + p.k) < lim && 2 * (32 * p.lda + p.k) < lim;
}

// The panel kernel (short K, A resident in registers along a row panel):
// A stored M x K, 0 < K <= 128, and N a whole number of 16-byte output units
// for its LDS-staged row-segment stores; on top of vec_ok.
bool panel_ok(const gemm_plan_t& p) {
  const int64_t units = p.out_type == TG_FP32 ? 4 : 8;
  return !p.trans_a && p.k > 0 && p.k <= tg::kPanelKMax && p.n % units == 0;
}

bool skinny_fits(int t, int64_t m) { return m <= 16 * kSkinny[t].mb; }

int skinny_choose(int64_t m, int64_t) { return m > 16 ? 1 : 0; }

// Tile choice by shape class and bound ("Optimize Triton Block Parameters",
// Step 1 roofline classification and shape-specific tuning; a small M wants a
// small BLOCK_M).  Work items are tiles times batch matrices.
//  * MFMA-bound problems (arithmetic intensity above MI355X's ~312 FLOP/B
//    ridge) take the 256x256 ping-pong kernel (8 waves alternating MFMA and
//    memory phases) from 128 work items on;
//  * HBM-bound ones with K <= 128 and >= 2048 tiles take the panel kernel
//    (runs of 128x128 tiles along a row panel of C: the next tile's B copy
//    overlaps this tile's stores);
//  * other HBM-bound ones take 256x128 tiles when N <= 256 (B panels read
//    half as often), else 128x128 tiles, two work-groups per CU, whose
//    operand panels and 1 KiB row-segment stores keep the streams long;
//  * small and ragged problems take 64x64 tiles so that there are at least
//    ~256 work-groups, with a 4-deep ring when K is long.
int choose_tile(const gemm_plan_t& p, int64_t batch) {
  const int64_t m = p.m, n = p.n, k = p.k;
  const int out_size = p.out_type == TG_FP32 ? 4 : 2;
  auto items = [&](int t) { return cdiv(m, kTiles[t].bm) * cdiv(n, kTiles[t].bn) * batch; };
  if (m <= 32) return tg::kThinTile;
  const double flops = 2.0 * (double)m * (double)n * (double)k;
  const double bytes = 2.0 * ((double)m * k + (double)k * n) + (double)out_size * m * n;
  const bool mfma_bound = bytes > 0 && flops / bytes > 312.5;
  // 256x256, 8 waves: from more than 128 work items on.  At exactly 128
  // (half the CUs) the 128x128 tiles with two work-groups per CU, one round of
  // 512, win at every K (8192x1024 and 2048x4096, K = 1024 .. 8192: 24 vs 31
  // us .. 128 vs 140 us); from 144 items on the ping-pong kernel does (3072^2
  // x 8192: 141 vs 196 us; 4096^2 x 8192: 0.204 vs 0.370 ms).
  if (mfma_bound && items(tg::kWideTile) > 128 && k > 0) return tg::kPingPongTile;
  // short K and many tiles: runs along row panels, A held in registers
  if (!mfma_bound && panel_ok(p) && items(tg::kPanelTile) >= 2048) return tg::kPanelTile;
  // HBM-bound with N <= 256: 256x128 tiles read each B panel half as often
  // as 128-row ones (128 x 2048x128x2048, fp32 out: 226 -> 205 us; 128 x
  // 512x128x8192: 286 -> 223 us; N = 64: 219 -> 201 us).  They need enough
  // work items (16384x128x16384, 64 of them: 229 -> 276 us) and rows.
  if (!mfma_bound && n <= 256 && m >= 256 && items(tg::kTallTile) >= 256) return tg::kTallTile;
  // 128x128, two work-groups per CU: HBM-bound products, and MFMA-bound ones
  // below the ping-pong kernel's range (measured faster than one work-group
  // per CU on every such shape tried: 1536x3072x8192 105 vs 173 us, 2560^2 x
  // 8192 117 vs 176 us, 2048^2 x 8192 88 vs 95 us)
  if (items(tg::kHbmTile) >= 256) return tg::kHbmTile;
  // MFMA-bound with more than 128 of them: still 128x128 (1536^2 x 8192: 84
  // vs 99 us on the 64x64 ring; at 128 items, 1024x2048x8192, 64x64 wins)
  if (mfma_bound && items(tg::kHbmTile) > 128) return tg::kHbmTile;
  // 64x64 tiles, at most one per CU: the four waves of a tile split its K
  // range (1000^3: 11.0 -> 10.4 us NN, 11.2 -> 9.7 us TN; 256^3: 5.5 -> 5.2 us)
  if (items(tg::kSmallTile) <= 256 && k >= 128) return tg::kKSliceTile;
  // more 64x64 tiles: with a long K the 4-deep ring keeps three steps'
  // copies in flight (1000^3: 12.3 -> 11.1 us); with a short one the 2-deep
  // ring's shorter prologue wins (256^3: 5.5 vs 5.9 us)
  return k >= 512 ? tg::kDeepSmallTile : tg::kSmallTile;
}

int choose_generic(int64_t m, int64_t n, int64_t batch) { return cdiv(m, 128) * cdiv(n, 128) * batch >= 256 ? 1 : 0; }

struct Launch {
  int bm, bn, bk, threads, stages, lds, dyn_lds;  // lds: total bytes; dyn_lds: dynamic part
};

Launch launch_shape(int variant, int tile) {
  if (variant == TG_VARIANT_SKINNY) {
    const tg::SkinnyShape& s = kSkinny[tile];
    return Launch{16 * s.mb, 16 * s.nb, s.sk, 64 * s.waves, s.stages, tg::skinny_lds_of(s), 0};
  }
  const TileShape& t = variant == TG_VARIANT_TILE ? kTiles[tile] : kGenericTiles[tile];
  return Launch{t.bm, t.bn, t.bk, 64 * t.wm * t.wn, t.stages, tg::lds_bytes_of(t), tg::lds_bytes_of(t)};
}

void fill_shape(gemm_plan_t* p) {
  const Launch l = launch_shape(p->variant, p->tile);
  p->bm = l.bm;
  p->bn = l.bn;
  p->bk = l.bk;
  p->wg_threads = l.threads;
  p->stages = l.stages;
  p->lds_bytes = (uint32_t)l.lds;
  p->tiles_m = p->variant == TG_VARIANT_SKINNY ? 1 : cdiv(p->m, p->bm);
  p->tiles_n = cdiv(p->n, p->bn);
  p->flags = (p->flags & ~TG_FLAG_EVEN_K) | ((p->bk > 0 && p->k % p->bk == 0) ? TG_FLAG_EVEN_K : 0);
  // Rotated K walks when no two tiles share an operand panel in the same
  // step (a single row or column of tiles): each work-group streams a panel
  // of its own, and lock-step walks would crowd the same HBM channels.
  const bool rotate = p->variant == TG_VARIANT_TILE && (p->tiles_m == 1 || p->tiles_n == 1);
  p->flags = (p->flags & ~TG_FLAG_ROTATE_K) | (rotate ? TG_FLAG_ROTATE_K : 0);
  // Persistent launches: work-groups that loop over tiles keep their CU
  // slot, where short-lived ones measured idle slots waiting for dispatch.
  // Prefetching the next tile during this tile's stores pays off where the
  // MFMA work per tile dwarfs its memory traffic; it stores straight from
  // registers, 4 columns at a time.  HBM-bound shapes keep the LDS-staged
  // row-segment stores, which measured faster for them.
  const double flops = 2.0 * (double)p->m * (double)p->n * (double)p->k;
  const double bytes = 2.0 * ((double)p->m * p->k + (double)p->k * p->n) +
                       (p->out_type == TG_FP32 ? 4.0 : 2.0) * (double)p->m * p->n;
  const bool persist = p->variant == TG_VARIANT_TILE;
  const bool prefetch = persist && p->n % 4 == 0 && bytes > 0 && flops / bytes > 312.5;
  p->flags = (p->flags & ~(TG_FLAG_PERSIST | TG_FLAG_PREFETCH)) | (persist ? TG_FLAG_PERSIST : 0) |
             (prefetch ? TG_FLAG_PREFETCH : 0);
  // TG_FLAG_STREAM_C is decided by bmm_plan, which knows the batch count
  p->flags &= ~TG_FLAG_STREAM_C;
}

}  // namespace

extern "C" {

const char* tg_status_str(tg_status s) {
  switch (s) {
    case TG_OK: return "ok";
    case TG_ERR_INVALID: return "invalid argument";
    case TG_ERR_UNSUPPORTED: return "unsupported";
    case TG_ERR_HIP: return "HIP launch error";
    case TG_ERR_TOO_LARGE: return "problem exceeds the fixed scratch array";
  }
  return "unknown status";
}

int32_t tg_abi_version(void) { return TG_ABI_VERSION; }

int32_t tg_variant_tiles(int32_t variant) {
  switch (variant) {
    case TG_VARIANT_GENERIC: return kNumGeneric;
    case TG_VARIANT_TILE: return kNumTiles;
    case TG_VARIANT_SKINNY: return kNumSkinny;
  }
  return 0;
}

tg_status bmm_plan(gemm_plan_t* plan, tg_dtype in_type, tg_dtype out_type, int trans_a, int trans_b, int64_t m,
                   int64_t n, int64_t k, int64_t lda, int64_t ldb, int64_t ldc, int64_t batch) {
  if (!plan) return TG_ERR_INVALID;
  if (batch < 1) {
    gemm_plan_t p = {};
    p.abi_version = -1;
    *plan = p;
    return TG_ERR_INVALID;
  }
  gemm_plan_t p = {};
  p.abi_version = -1;
  *plan = p;
  if (m < 0 || n < 0 || k < 0) return TG_ERR_INVALID;
  if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return TG_ERR_INVALID;
  const int64_t lim = (int64_t)1 << 31;
  if (m >= lim || n >= lim || k >= lim) return TG_ERR_INVALID;
  const int64_t min_lda = trans_a ? m : k, min_ldb = trans_b ? k : n;
  if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) || ldc < (n > 1 ? n : 1))
    return TG_ERR_INVALID;
  // element offsets of every operand must stay far inside int64
  const int64_t big = (int64_t)1 << 60;
  if (lda > big / ((trans_a ? k : m) + 1) || ldb > big / ((trans_b ? n : k) + 1) || ldc > big / (m + 1))
    return TG_ERR_INVALID;
  if (in_type != TG_BF16 && in_type != TG_FP16) return TG_ERR_UNSUPPORTED;
  if (out_type != TG_FP32 && out_type != in_type) return TG_ERR_UNSUPPORTED;

  p.in_type = in_type;
  p.out_type = out_type;
  p.trans_a = trans_a;
  p.trans_b = trans_b;
  p.m = m;
  p.n = n;
  p.k = k;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.workspace_bytes = 0;
  p.flags = vec_ok(p) ? TG_FLAG_VEC16 : 0;
  if (skinny_ok(p)) {
    p.variant = TG_VARIANT_SKINNY;
    p.tile = skinny_choose(m, n);
  } else if (p.flags & TG_FLAG_VEC16) {
    p.variant = TG_VARIANT_TILE;
    p.tile = choose_tile(p, batch);
  } else {
    p.variant = TG_VARIANT_GENERIC;
    p.tile = choose_generic(m, n, batch);
  }
  fill_shape(&p);
  if (p.tiles_m * p.tiles_n >= lim) return TG_ERR_INVALID;
  // Non-temporal C stores when one launch writes far more than the L2s hold
  // (8 x 4 MiB): measured 16% faster on the 2 GiB attention-score product,
  // whose store stream otherwise evicts the Q and K panels the tiles re-read.
  if (p.variant == TG_VARIANT_TILE &&
      (double)m * (double)n * (double)batch * (out_type == TG_FP32 ? 4.0 : 2.0) >= 64.0 * (1 << 20))
    p.flags |= TG_FLAG_STREAM_C;
  p.abi_version = TG_ABI_VERSION;
  *plan = p;
  return TG_OK;
}

tg_status gemm_plan(gemm_plan_t* plan, tg_dtype in_type, tg_dtype out_type, int trans_a, int trans_b, int64_t m,
                    int64_t n, int64_t k, int64_t lda, int64_t ldb, int64_t ldc) {
  return bmm_plan(plan, in_type, out_type, trans_a, trans_b, m, n, k, lda, ldb, ldc, 1);
}

tg_status gemm_plan_tile(gemm_plan_t* plan, int32_t variant, int32_t tile) {
  if (!plan || plan->abi_version != TG_ABI_VERSION) return TG_ERR_INVALID;
  gemm_plan_t p = *plan;
  if (variant == TG_VARIANT_SKINNY) {
    if (tile < 0 || tile >= kNumSkinny || !skinny_ok(p) || !skinny_fits(tile, p.m)) return TG_ERR_UNSUPPORTED;
  } else if (variant == TG_VARIANT_TILE) {
    if (tile < 0 || tile >= kNumTiles || !vec_ok(p)) return TG_ERR_UNSUPPORTED;
  } else if (variant == TG_VARIANT_GENERIC) {
    if (tile < 0 || tile >= kNumGeneric) return TG_ERR_UNSUPPORTED;
  } else {
    return TG_ERR_UNSUPPORTED;
  }
  const int32_t stream_c = p.flags & TG_FLAG_STREAM_C;  // bmm_plan's choice (it knew the batch)
  p.variant = variant;
  p.tile = tile;
  fill_shape(&p);
  if (variant == TG_VARIANT_TILE) p.flags |= stream_c;
  if (p.tiles_m * p.tiles_n >= ((int64_t)1 << 31)) return TG_ERR_UNSUPPORTED;
  *plan = p;
  return TG_OK;
}

// Compute units of the current device, cached per device (the value never
// changes; racing first calls store the same number).
static int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

static tg_status launch(const gemm_plan_t* plan, const gemm_epilogue_t* epi, int64_t batch, int64_t sA, int64_t sB,
                        int64_t sC, const void* A, const void* B, void* C, hipStream_t stream) {
  if (!plan || plan->abi_version != TG_ABI_VERSION) return TG_ERR_INVALID;
  if (batch < 0 || sA < 0 || sB < 0 || sC < 0) return TG_ERR_INVALID;
  const gemm_plan_t& p = *plan;
  if (p.m == 0 || p.n == 0 || batch == 0) return TG_OK;
  if (!C) return TG_ERR_INVALID;
  if (p.k > 0 && (!A || !B)) return TG_ERR_INVALID;
  if (p.in_type < 0 || p.in_type > 1 || (p.out_type != TG_FP32 && p.out_type != p.in_type)) return TG_ERR_INVALID;
  if (batch > 1 && sC < (p.m - 1) * p.ldc + p.n) return TG_ERR_INVALID;  // batches' outputs would overlap

  // re-validate the (variant, tile) pair: callers may override it
  int variant = p.variant, tile = p.tile;
  if (variant == TG_VARIANT_SKINNY) {
    if (tile < 0 || tile >= kNumSkinny || !skinny_ok(p) || !skinny_fits(tile, p.m)) return TG_ERR_UNSUPPORTED;
  } else if (variant == TG_VARIANT_TILE) {
    if (tile < 0 || tile >= kNumTiles || !vec_ok(p)) return TG_ERR_UNSUPPORTED;
  } else if (variant == TG_VARIANT_GENERIC) {
    if (tile < 0 || tile >= kNumGeneric) return TG_ERR_UNSUPPORTED;
  } else {
    return TG_ERR_UNSUPPORTED;
  }
  // vector paths need 16-byte aligned bases and batch strides; else gather element-wise
  const bool aligned = ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0) && ((uintptr_t)C % 16 == 0) &&
                       (batch == 1 || (sA % 8 == 0 && sB % 8 == 0 && sC % 8 == 0));
  if (variant != TG_VARIANT_GENERIC && !aligned) {
    variant = TG_VARIANT_GENERIC;
    tile = choose_generic(p.m, p.n, batch);
  }

  tg::GemmArgs a;
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.C = C;
  a.M = p.m;
  a.N = p.n;
  a.K = p.k;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldc = p.ldc;
  a.sA = sA;
  a.sB = sB;
  a.sC = sC;
  a.batch = batch;
  a.rotate_k = (variant == TG_VARIANT_TILE && (p.flags & TG_FLAG_ROTATE_K)) ? 1 : 0;
  a.persist = 0;
  // an identity epilogue (alpha 1, beta 0, no bias) is no epilogue
  a.epi = epi && !(epi->alpha == 1.f && epi->beta == 0.f && !epi->bias) ? 1 : 0;
  a.alpha = epi ? epi->alpha : 1.f;
  a.beta = epi ? epi->beta : 0.f;
  a.bias = epi ? epi->bias : nullptr;
  a.stream_c = (variant == TG_VARIANT_TILE && (p.flags & TG_FLAG_STREAM_C)) ? 1 : 0;
  if (a.epi && a.bias && (uintptr_t)a.bias % (p.out_type == TG_FP32 ? 4 : 2) != 0) return TG_ERR_INVALID;

  // The ping-pong kernel: its epilogue entry when there is an epilogue; the
  // 8-wave tile kernel for K = 0 (which it does not handle) and for more
  // items than its 32-bit item order covers.
  const bool pingpong = variant == TG_VARIANT_TILE &&
                        (kTiles[tile].kind == tg::kPingPong || kTiles[tile].kind == tg::kPingPongEpi);
  if (pingpong) {
    const int64_t items = cdiv(p.m, kTiles[tile].bm) * cdiv(p.n, kTiles[tile].bn) * batch;
    // (its 32-bit step counters: items x K steps below 2^31)
    if (p.k == 0 || items >= ((int64_t)1 << 30) || items * cdiv(p.k, kTiles[tile].bk) >= ((int64_t)1 << 31))
      tile = tg::kWideTile;
    else
      tile = a.epi ? tg::kPingPongEpiTile : tg::kPingPongTile;
  }
  // The panel kernel; what it does not serve goes to the 128 x 128 tile.
  if (variant == TG_VARIANT_TILE && kTiles[tile].kind == tg::kPanel && (a.epi || !panel_ok(p))) tile = tg::kHbmTile;
  // The tile kernel's entries leave the epilogue out; a call with one goes
  // to the entry of the same shape class that has it compiled in.
  if (variant == TG_VARIANT_TILE && a.epi && kTiles[tile].kind == tg::kTileKernel) tile = tg::epi_twin(tile);
  a.span = 0;
  // Tile kernel: an operand that only one tile of the launch reads -- A when
  // there is one column of tiles, B when there is one row, and neither when
  // a zero batch stride shares it between matrices -- streams through the
  // L2 with non-temporal loads (measured 8% faster on O = P V, whose P rows
  // otherwise evict the V panel the 16 row blocks of a head share).
  a.nt_ab = 0;
  if (variant == TG_VARIANT_TILE && (kTiles[tile].kind == tg::kTileKernel || kTiles[tile].kind == tg::kTileEpi)) {
    const int64_t tm = cdiv(p.m, kTiles[tile].bm), tn = cdiv(p.n, kTiles[tile].bn);
    if (tn == 1 && (batch == 1 || sA != 0)) a.nt_ab |= 1;
    if (tm == 1 && (batch == 1 || sB != 0)) a.nt_ab |= 2;
  }
  const Launch l = launch_shape(variant, tile);
  const int io = p.in_type == TG_BF16 ? 0 : 1, oo = p.out_type == TG_FP32 ? 0 : 1;
  KernelFn fn;
  if (variant == TG_VARIANT_SKINNY) {
    a.tiles_m = 1;
    a.tiles_n = (int32_t)cdiv(p.n, l.bn);
    fn = tg::skinny_table[io][oo][tile];
  } else {
    a.tiles_m = (int32_t)cdiv(p.m, l.bm);
    a.tiles_n = (int32_t)cdiv(p.n, l.bn);
    const int tr = 2 * p.trans_a + p.trans_b;
    fn = variant == TG_VARIANT_TILE ? kTileTables[io][oo][tr][tile] : kGenericTables[io][oo][tr][tile];
  }
  const int64_t groups = (int64_t)a.tiles_m * a.tiles_n;
  if (groups >= ((int64_t)1 << 31)) return TG_ERR_INVALID;
  dim3 grid;
  if (variant == TG_VARIANT_SKINNY) {
    grid = dim3((unsigned)groups, (unsigned)(batch < 65535 ? batch : 65535));
  } else {
    // one work-group per (matrix, tile) work item, flattened; beyond 2^30
    // items each work-group loops (the stride stays a multiple of 8, which
    // keeps every item on the XCD the kernel's tile order assumes)
    int64_t total = groups * batch;
    int64_t cap = (int64_t)1 << 30;
    if (variant == TG_VARIANT_TILE && kTiles[tile].kind == tg::kPanel) {
      // one work-group per run of column tiles: whole row panels, halved
      // while there are fewer than 4 runs per CU (down to 4 tiles a run)
      const int64_t target = 4 * (int64_t)compute_units();
      int32_t span = a.tiles_n;
      while (span > 4 && batch * a.tiles_m * cdiv(a.tiles_n, span) < target) span = (span + 1) / 2;
      a.span = span;
      total = batch * a.tiles_m * cdiv(a.tiles_n, span);
    } else if (variant == TG_VARIANT_TILE && kTiles[tile].kind == tg::kPingPong) {
      // persistent ping-pong: one work-group per CU; it stores each finished
      // tile with 4-column vector stores (N % 4 == 0) and has no epilogue
      const int64_t slots = (int64_t)compute_units();
      if ((p.flags & TG_FLAG_PERSIST) && p.n % 4 == 0 && slots > 0 && total >= 2 * slots) cap = slots;
    } else if (variant == TG_VARIANT_TILE && (p.flags & TG_FLAG_PERSIST) && !a.epi) {
      // persistent: one work-group per resident slot (a multiple of 8)
      const int64_t slots = (int64_t)compute_units() * kTiles[tile].occ;
      if (slots > 0 && total >= 2 * slots) {
        cap = slots;
        if ((p.flags & TG_FLAG_PREFETCH) && p.n % 4 == 0 && tg::persist_ok(kTiles[tile]))
          a.persist = 1;  // every wave prefetches, then stores from registers
      }
    }
    grid = dim3((unsigned)(total < cap ? total : cap), 1);
  }
  if (l.dyn_lds > 64 * 1024) {
    if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, l.dyn_lds) != hipSuccess)
      return TG_ERR_HIP;
  }
  hipLaunchKernelGGL(fn, grid, dim3(l.threads), (size_t)l.dyn_lds, stream, a);
  return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

int32_t tg_group_tiles(void) { return kNumGroup; }

// Grouped launch.  Each problem is validated by gemm_plan; every check runs
// before anything is enqueued.  Problems the vector loader cannot serve run
// one by one through gemm_run (element-wise loader); the others go out in
// launches of up to TG_GROUP_MAX problems, in the order given.
tg_status gemm_group_run(tg_dtype in_type, tg_dtype out_type, int trans_a, int trans_b,
                         const gemm_group_problem_t* problems, int64_t count, int32_t tile, hipStream_t stream) {
  if (count < 0 || (count > 0 && !problems)) return TG_ERR_INVALID;
  if (tile < -1 || tile >= kNumGroup) return TG_ERR_UNSUPPORTED;
  for (int64_t i = 0; i < count; ++i) {
    const gemm_group_problem_t& q = problems[i];
    gemm_plan_t p;
    const tg_status st = gemm_plan(&p, in_type, out_type, trans_a, trans_b, q.m, q.n, q.k, q.lda, q.ldb, q.ldc);
    if (st != TG_OK) return st;
    if (q.m > 0 && q.n > 0 && (!q.C || (q.k > 0 && (!q.A || !q.B)))) return TG_ERR_INVALID;
    if (cdiv(q.m, 64) * cdiv(q.n, 64) >= ((int64_t)1 << 30)) return TG_ERR_INVALID;  // item count must fit int32
  }
  const int io = in_type == TG_BF16 ? 0 : 1, oo = out_type == TG_FP32 ? 0 : 1, tr = 2 * trans_a + trans_b;
  const int out_size = out_type == TG_FP32 ? 4 : 2;

  tg::GroupArgs g;
  g.g = tg::GemmArgs{};
  g.count = 0;
  int64_t chunk_first[tg::kGroupMax];  // index into `problems` of each table entry
  auto flush = [&]() -> tg_status {
    if (g.count == 0) return TG_OK;
    // tile: by the group's totals, as choose_tile does for one problem
    int gt = tile;
    if (gt < 0) {
      double flops = 0, bytes = 0;
      int64_t max_m = 0;
      auto items = [&](int t) {
        int64_t n = 0;
        for (int i = 0; i < g.count; ++i) {
          const gemm_group_problem_t& q = problems[chunk_first[i]];
          n += cdiv(q.m, kTiles[t].bm) * cdiv(q.n, kTiles[t].bn);
        }
        return n;
      };
      for (int i = 0; i < g.count; ++i) {
        const gemm_group_problem_t& q = problems[chunk_first[i]];
        flops += 2.0 * (double)q.m * (double)q.n * (double)q.k;
        bytes += 2.0 * ((double)q.m * q.k + (double)q.k * q.n) + (double)out_size * q.m * q.n;
        max_m = q.m > max_m ? q.m : max_m;
      }
      const bool mfma_bound = bytes > 0 && flops / bytes > 312.5;
      // 128x128 tiles: for HBM-bound groups the 3-deep 32-wide ring with
      // three work-groups per CU (more copies in flight per CU; measured 4%
      // faster than two work-groups of 64-deep steps on 32 ragged experts)
      gt = 0;  // 64x64
      if (max_m > 32) {
        if (mfma_bound && items(tg::kWideTile) >= 512) gt = 3;       // 256x256, 8 waves
        else if (items(tg::kHbmTile) >= 256) gt = mfma_bound ? 2 : 4;
      }
    }
    const TileShape& t = kTiles[kGroupTiles[gt]];
    int64_t total = 0;
    for (int i = 0; i < g.count; ++i) {
      const gemm_group_problem_t& q = problems[chunk_first[i]];
      g.p[i].first = (int32_t)total;
      total += cdiv(q.m, t.bm) * cdiv(q.n, t.bn);
      if (total >= ((int64_t)1 << 31)) return TG_ERR_INVALID;
    }
    g.total = (int32_t)total;
    const tg::GroupFn fn = kGroupTables[io][oo][tr][gt];
    const int lds = tg::lds_bytes_of(t);
    if (lds > 64 * 1024) {
      if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return TG_ERR_HIP;
    }
    const int64_t cap = (int64_t)1 << 30;
    hipLaunchKernelGGL(fn, dim3((unsigned)(total < cap ? total : cap)), dim3(64 * t.wm * t.wn), (size_t)lds, stream,
                       g);
    g.count = 0;
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
  };

  for (int64_t i = 0; i < count; ++i) {
    const gemm_group_problem_t& q = problems[i];
    if (q.m == 0 || q.n == 0) continue;
    gemm_plan_t p;
    (void)gemm_plan(&p, in_type, out_type, trans_a, trans_b, q.m, q.n, q.k, q.lda, q.ldb, q.ldc);
    const bool aligned = (uintptr_t)q.C % 16 == 0 && (q.k == 0 || ((uintptr_t)q.A % 16 == 0 && (uintptr_t)q.B % 16 == 0));
    if (!(p.flags & TG_FLAG_VEC16) || !aligned || q.m > INT32_MAX || q.n > INT32_MAX || q.k > INT32_MAX) {
      const tg_status st = gemm_run(&p, q.A, q.B, q.C, stream);
      if (st != TG_OK) return st;
      continue;
    }
    tg::GroupProblem& e = g.p[g.count];
    e.A = static_cast<const uint16_t*>(q.A);
    e.B = static_cast<const uint16_t*>(q.B);
    e.C = q.C;
    e.lda = q.lda;
    e.ldb = q.ldb;
    e.ldc = q.ldc;
    e.M = (int32_t)q.m;
    e.N = (int32_t)q.n;
    e.K = (int32_t)q.k;
    chunk_first[g.count] = i;
    if (++g.count == tg::kGroupMax) {
      const tg_status st = flush();
      if (st != TG_OK) return st;
    }
  }
  return flush();
}

tg_status gemm_run(const gemm_plan_t* plan, const void* A, const void* B, void* C, hipStream_t stream) {
  return launch(plan, nullptr, 1, 0, 0, 0, A, B, C, stream);
}

tg_status bmm_run(const gemm_plan_t* plan, int64_t batch, int64_t stride_a, int64_t stride_b, int64_t stride_c,
                  const void* A, const void* B, void* C, hipStream_t stream) {
  return launch(plan, nullptr, batch, stride_a, stride_b, stride_c, A, B, C, stream);
}

tg_status gemm_run_ex(const gemm_plan_t* plan, const gemm_epilogue_t* epi, const void* A, const void* B, void* C,
                      hipStream_t stream) {
  return launch(plan, epi, 1, 0, 0, 0, A, B, C, stream);
}

tg_status bmm_run_ex(const gemm_plan_t* plan, const gemm_epilogue_t* epi, int64_t batch, int64_t stride_a,
                     int64_t stride_b, int64_t stride_c, const void* A, const void* B, void* C, hipStream_t stream) {
  return launch(plan, epi, batch, stride_a, stride_b, stride_c, A, B, C, stream);
}

}  // extern "C"
