// pingpong_gemm.hpp -- gfx950 GEMM/BMM for large MFMA-bound products: eight
// waves that alternate between a matrix-core phase and a memory phase.
//
// A work-group computes 256 x 256 tiles of C[b] = op(A[b]) op(B[b]) with
// eight waves in two groups of four.  Wave w runs on SIMD w mod 4, so every
// SIMD holds one wave of each group; a wave of group g owns rows
// [128 g, 128 g + 128) and columns [64 s, 64 s + 64) of the tile (s = w mod 4).
// The groups take turns, one work-group barrier per turn:
//
//   phase 2k   : group 0 reads its fragments of K step k from LDS (and
//                issues the HBM->LDS copies of step k + 1); group 1 runs the
//                MFMAs of step k - 1.
//   phase 2k+1 : group 0 runs the MFMAs of step k; group 1 reads its
//                fragments of step k.
//
// So on every SIMD one wave issues nothing but back-to-back MFMAs on
// fragments already in its registers while the other wave waits on LDS and
// HBM, and the matrix core idles only at the turn.  A turn's MFMAs (32
// blocks of 16 x 16, two 32-deep slices) outlast the other group's LDS reads.  This
// is the pages' producer/consumer split ("FLA Triton -> Gluon Porting
// Skill", section 5: warp-specialised pipelines) expressed with the two waves
// that share a SIMD.
//
//  * v_mfma_f32_16x16x32: measured under the power cap on random bf16
//    operands, it sustains ~7% more throughput than the 32x32x16 form (it
//    moves half the accumulator data per flop).
//  * Staging, op() by addressing and the zero-filled tails are the tile
//    kernel's (direct-to-LDS copies, ds_read_b64_tr_b16 for M/N-contiguous
//    operands), with a swizzle for M/N-contiguous tiles that suits the
//    16x16x32 transposing reads, and the addressing folded into a few
//    registers: a wave holds 128 accumulators and 96 fragment registers of
//    256.
//  * Ring: two LDS buffers of one 64-deep K step (2 x 64 KiB).  Step k + 1
//    goes into the buffer of step k - 1, which group 1 finished reading
//    before the barrier that opens phase 2k.  Group 0 waits for its copies of
//    step k + 1 at the end of its MFMA phase 2k+1, before the barrier that
//    opens phase 2k+2, where it reads step k + 1.
//  * Persistent: a work-group takes items blockIdx.x, blockIdx.x + gridDim.x,
//    ... (the XCD-aware order of work_coords), and their K steps form one
//    stream -- the copies of an item's first step are issued during the
//    previous item's last step like any other.  Each group stores a finished
//    item from registers at the start of its next memory phase, while the
//    other group runs MFMAs; the first step of an item starts its MFMAs from
//    zero accumulators.
#pragma once

#include "tile_gemm.hpp"

namespace tg {

// LDS swizzle of the ping-pong kernel, in 16-byte units.  K-contiguous tiles
// (rows of 64 elements) use the tile kernel's (row / 2) mod 8.  M/N-
// contiguous tiles (rows along K, 256 elements) flip the unit index by
// 2 * (bits 0-1 of the row, plus bit 3 of the row as bit 2): the transposing
// reads of the 16x16x32 fragments put rows k..k+3 and k+8..k+11 in one LDS
// clock, and these eight rows then land on eight distinct unit pairs.
template <bool KC, int CH>
__device__ __forceinline__ uint32_t pp_swz(uint32_t row) {
  if constexpr (KC)
    return swz_unit<true, CH>(row);
  else
    return (2u * ((row & 3u) | ((row >> 1) & 4u))) & (uint32_t)(CH - 1);
}
template <bool KC, int CH>
__device__ __forceinline__ uint32_t pp_off(uint32_t row, uint32_t col) {
  return row * (CH * 16u) + (((col >> 3) ^ pp_swz<KC, CH>(row)) << 4) + ((col & 7u) << 1);
}

// HBM->LDS copies of one operand's K step, issued by NW waves: lane t of a
// wave's instruction i writes LDS bytes (wave * IPW + i) KiB + 16 t, and
// fetches the source unit that the swizzle puts there.  Instruction i lands
// RPI tile rows below instruction i - 1, and the swizzle of its source units
// depends on i only through the bits in BMASK, so a wave's source offsets
// are a few per-lane bases plus multiples of one uniform row stride (two or
// four registers instead of one per instruction).
template <bool KC, int MN_T, int BK, int NW>
struct DmaPair {
  static constexpr int CH = KC ? BK / 8 : MN_T / 8;
  static constexpr int BYTES = MN_T * BK * 2;
  static constexpr int INSTR = BYTES / 1024;
  static constexpr int IPW = INSTR / NW;
  static constexpr int RPI = 1024 / (CH * 16);  // tile rows per instruction
  // K-contiguous: the swizzle sees (row / 2) mod 8, i.e. instruction parity;
  // M/N-contiguous (two rows per instruction): row bits 1 and 3, i.e.
  // instruction bits 0 and 2
  static constexpr int BMASK = KC ? 1 : 5;
  static constexpr int NB = KC ? 2 : 4;
  static_assert(KC ? CH == 8 : CH == 32, "64-deep K-contiguous rows or 256-wide M/N-contiguous rows");
  static_assert(BYTES % 1024 == 0 && INSTR % NW == 0 && IPW % 8 == 0, "whole 1 KiB wave loads");

  uint32_t vb[NB];  // source byte offsets of the base instructions

  static __device__ __forceinline__ int slot(int i) { return KC ? (i & 1) : ((i & 1) | ((i >> 1) & 2)); }
  static __device__ __forceinline__ uint32_t unit_of(int wave, int lane, int i, uint32_t& row) {
    const uint32_t o = (uint32_t)(wave * IPW + i) * 1024u + 16u * lane;
    row = o / (CH * 16);
    return ((o / 16) % CH) ^ pp_swz<KC, CH>(row);
  }
  __device__ __forceinline__ void init(int wave, int lane, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & BMASK) != i) continue;
      uint32_t row;
      const uint32_t unit = unit_of(wave, lane, i, row);
      vb[slot(i)] = row * (uint32_t)ld * 2u + unit * 16u;
    }
  }
  // keep the bases in registers (the compiler would rather recompute them
  // in the loop, which costs issue slots in the memory phase)
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int b = 0; b < NB; ++b) asm volatile("" : "+v"(vb[b]));
  }

  // base: element (mn0, k0) [KC] or (k0, mn0) [MN]; bytes: from base to the
  // end of the matrix's last element; k_left = K - k0 (units at or past K
  // of a K-contiguous tile read zero when MASK_K).
  template <bool MASK_K>
  __device__ __forceinline__ void issue(const uint16_t* base, int64_t bytes, int64_t ld, uint32_t tile_lds, int wave,
                                        int lane, int64_t k_left) const {
    const i32x4 rs = make_rsrc(base, bytes);
    const uint32_t row_bytes = (uint32_t)RPI * (uint32_t)ld * 2u;
    const int32_t kl = k_left < BK ? (int32_t)k_left : BK;
    uint32_t ln = lane;
    if constexpr (MASK_K && KC) asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));  // (not hoisted)
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int bi = i & BMASK;
      uint32_t off = vb[slot(bi)] + (uint32_t)(i - bi) * row_bytes;
      if constexpr (MASK_K && KC) {
        uint32_t row;
        const uint32_t kofs = unit_of(wave, ln, i, row) * 8;
        off = (int32_t)kofs < kl ? off : kOutOfRange;
      }
      dma16(rs, off, tile_lds + (uint32_t)(wave * IPW + i) * 1024u);
    }
  }
};

// LDS byte offsets of a wave's 16x16x32 MFMA fragments: lane l supplies
// row/column (l & 15) of a 16-wide block and the 8 consecutive k at
// 8 (l >> 4) of a 32-deep slice.  K-contiguous tiles (rows of 64 elements,
// CH = 8): a block 16 rows down is 2 KiB further, and slice ks flips bit 6
// of the slice-0 offset (the swizzle XORs whole units).  M/N-contiguous
// tiles (rows of 256 elements, CH = 32) are read with two transposing reads
// of 4 k-rows each: a block 16 columns over flips bits 5-6, a slice is 32
// rows (16 KiB) further and the second read 4 rows (2 KiB).  So one
// register serves every fragment of an operand.
template <bool KC, int CH>
struct FragAddr {
  uint32_t r;
  __device__ __forceinline__ void init(int mn0, int lane) {
    const int i = lane & 15, h = lane >> 4;
    if constexpr (KC)
      r = pp_off<true, CH>(mn0 + i, 8 * h);
    else
      r = pp_off<false, CH>(8 * h + (i >> 2), mn0 + 4 * (i & 3));
  }
  __device__ __forceinline__ void pin() { asm volatile("" : "+v"(r)); }
  __device__ __forceinline__ uint32_t at(int ks, int b) const {
    if constexpr (KC)
      return (r ^ (uint32_t)(ks << 6)) + (uint32_t)b * 16u * CH * 16u;
    else
      return (r ^ (uint32_t)(b << 5)) + (uint32_t)ks * 32u * CH * 16u;
  }
  static constexpr uint32_t TR4 = 4u * CH * 16u;  // second transposing read: 4 rows down
};

// A wave's result is FM x FN blocks of 16 x 16 (v_mfma_f32_16x16x32 with the
// B fragment as the first operand): register q of block (i, j) of lane l is
// C[16 i + (l & 15)][16 j + 4 (l >> 4) + q] relative to the wave's corner --
// four consecutive columns of one row.

// Vector store of the blocks, exactly FM * FN store instructions.  Column
// offsets inside the wave's tile are instruction immediates; when the tile
// ends inside the blocks (n_left < FN * 16) whole 4-column groups at or past
// n_left are dropped (the caller guarantees N % 4 == 0 or a tile that ends
// inside N).  Rows past the descriptor's end are dropped.  Each group is
// converted right before its store, so only two temporaries are live
// besides the accumulators.
template <typename Out, int FM, int FN>
__device__ __forceinline__ void store16_vec(const void* Ctile, int64_t bytes, int64_t ldc, int64_t n_left, int lane,
                                            const f32x4 (&acc)[FM][FN]) {
  const __amdgpu_buffer_rsrc_t rs = store_rsrc(Ctile, bytes);
  // an opaque copy of the lane index keeps the compiler from hoisting the
  // row offsets and column masks out of the caller's loop (and spilling them)
  uint32_t ln;
  asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
  const uint32_t lr = ln & 15u, lc = 4u * (ln >> 4);
  constexpr uint32_t es = sizeof(Out);
  const bool full = n_left >= FN * 16;
  const int32_t nl = n_left < FN * 16 ? (int32_t)n_left : FN * 16;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const uint32_t rowoff = (16u * i + lr) * (uint32_t)ldc * es + lc * es;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint32_t col = (uint32_t)(16 * j);
      const uint32_t off = (full || (int32_t)(col + lc) < nl) ? rowoff + col * es : kOutOfRange;
      const f32x4& a = acc[i][j];
      if constexpr (es == 4)
        buf_store16(rs, off, __builtin_bit_cast(u32x4, a));
      else
        buf_store8(rs, off, u32x2{pack2<Out>(a[0], a[1]), pack2<Out>(a[2], a[3])});
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Element-wise store with bounds checks (any N, any alignment of ldc).
template <typename Out, int FM, int FN>
__device__ __forceinline__ void store16_elem(void* Cb, int64_t ldc, int64_t M, int64_t N, int64_t r0, int64_t c0,
                                             int lane, const f32x4 (&acc)[FM][FN]) {
  const int lr = lane & 15, lc = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = r0 + 16 * i + lr;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = c0 + 16 * j + lc + q;
        if (row < M && col < N) store_out<Out>(Cb, row * ldc + col, acc[i][j][q]);
      }
  }
}

// acc = alpha * acc + beta * C + bias[col] in fp32 (C read only if beta != 0;
// entries outside M x N are left alone and never stored).
template <typename Out, int FM, int FN>
__device__ __forceinline__ void epilogue16(const GemmArgs& args, const void* Cb, int64_t ldc, int64_t M, int64_t N,
                                           int64_t r0, int64_t c0, int lane, f32x4 (&acc)[FM][FN]) {
  const int lr = lane & 15, lc = 4 * (lane >> 4);
  const float alpha = args.alpha, beta = args.beta;
  const bool use_c = beta != 0.f, use_bias = args.bias != nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = r0 + 16 * i + lr;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = c0 + 16 * j + lc + q;
        float v = alpha * acc[i][j][q];
        if (row < M && col < N) {
          if (use_c) v = __builtin_fmaf(beta, load_out<Out>(Cb, row * ldc + col), v);
          if (use_bias) v += load_out<Out>(args.bias, col);
        }
        acc[i][j][q] = v;
      }
  }
}

template <typename In, typename Out, bool TA, bool TB, bool EPI>
__global__ void __launch_bounds__(512, 1) pingpong_gemm_kernel(GemmArgs args) {
  constexpr int BM = 256, BN = 256, BK = 64, WN = 4;
  constexpr int WTM = 128, WTN = 64, FM = WTM / 16, FN = WTN / 16, KS = BK / 32;
  constexpr bool A_KC = !TA, B_KC = TB;
  using OA = DmaPair<A_KC, BM, BK, 4>;  // issued by the four waves of group 1
  using OB = DmaPair<B_KC, BN, BK, 4>;  // issued by the four waves of group 0
  constexpr uint32_t A_BYTES = OA::BYTES, B_BYTES = OB::BYTES;
  constexpr uint32_t B_BASE = 3 * A_BYTES;  // three A buffers, then two B buffers
  constexpr int PA = OA::IPW, PB = OB::IPW;  // copy instructions per wave per step
  constexpr int ST = FM * FN;                // store instructions of store16_vec
  static_assert(B_BASE + 2 * B_BYTES <= 160 * 1024, "LDS budget");
  static_assert(PA + ST < 64 && PB + ST < 64, "counted waits fit the vector-memory counter");

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;
  const uint32_t lds0 = (uint32_t)(size_t)lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave / WN, sw = wave % WN;
  const int wm0 = grp * WTM, wn0 = sw * WTN;

  const int64_t M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb, ldc = args.ldc;
  const int64_t total = (int64_t)args.tiles_m * args.tiles_n * args.batch;
  if ((int64_t)blockIdx.x >= total || K <= 0) return;  // (the launcher never sends K = 0 here)
  // This work-group's items are blockIdx.x, blockIdx.x + gridDim.x, ...; their
  // K steps form one stream of nsteps steps (the launcher keeps the launch's
  // item count times nk below 2^31, so 32-bit counters do).
  const int32_t nk = (int32_t)((K + BK - 1) / BK);
  const int32_t items = (int32_t)((total - 1 - (int64_t)blockIdx.x) / gridDim.x + 1);
  const int32_t nsteps = items * nk;
  const bool k_ragged = K % BK != 0;  // the last step of each item is masked

  struct Item {
    int64_t b, m0, n0;
  };
  // item t of this work-group: work_coords' XCD-aware order in 32-bit
  // arithmetic (the launcher keeps total below 2^31)
  auto item_of = [&](int32_t t) {
    const uint32_t tot = (uint32_t)total, tm = (uint32_t)args.tiles_m, tn = (uint32_t)args.tiles_n;
    const uint32_t w0 = blockIdx.x + (uint32_t)t * gridDim.x;
    const uint32_t per = tot >> 3, rem = tot & 7, x = w0 & 7, local = w0 >> 3;
    const uint32_t id = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
    const uint32_t G = tm * tn, bb = id / G, tt = id - bb * G;
    const uint32_t band = 8 * tn, bidx = tt / band, first_m = bidx * 8;
    const uint32_t gsz = min(tm - first_m, 8u), in_band = tt - bidx * band;
    Item it;
    it.b = bb;
    it.m0 = (int64_t)(first_m + in_band % gsz) * BM;
    it.n0 = (int64_t)(in_band / gsz) * BN;
    return it;
  };

  // Copy cursor of one operand: the next step it copies, as (item, step in
  // item), with the source of that step and the bytes from there to the end
  // of the matrix.  Advancing within an item is two 64-bit adds; only a new
  // item recomputes its panel origin.
  struct Cursor {
    int32_t t, k;
    const char* ptr;
    int64_t left;
  };
  const int64_t a_step = A_KC ? (int64_t)BK * 2 : (int64_t)BK * lda * 2;
  const int64_t b_step = B_KC ? (int64_t)BK * 2 : (int64_t)BK * ldb * 2;
  auto a_seek = [&](Cursor& c) {
    const Item it = item_of(c.t);
    const int64_t o = (int64_t)c.k * a_step;
    c.ptr = (const char*)(args.A + it.b * args.sA + (A_KC ? it.m0 * lda : it.m0)) + o;
    c.left = (A_KC ? ((M - 1 - it.m0) * lda + K) * 2 : ((K - 1) * lda + (M - it.m0)) * 2) - o;
  };
  auto b_seek = [&](Cursor& c) {
    const Item it = item_of(c.t);
    const int64_t o = (int64_t)c.k * b_step;
    c.ptr = (const char*)(args.B + it.b * args.sB + (B_KC ? it.n0 * ldb : it.n0)) + o;
    c.left = (B_KC ? ((N - 1 - it.n0) * ldb + K) * 2 : ((K - 1) * ldb + (N - it.n0)) * 2) - o;
  };
  OA oa;
  OB ob;
  oa.init(sw, lane, lda);
  ob.init(sw, lane, ldb);
  // copy the cursor's step into buffer `buf`, then advance the cursor (the
  // last step of an item is masked at K when K is not a multiple of BK)
  auto copy_a = [&](Cursor& c, uint32_t buf) {
    const uint32_t dst = lds0 + buf * A_BYTES;
    if (k_ragged && c.k == nk - 1)
      oa.template issue<true>((const uint16_t*)c.ptr, c.left, lda, dst, sw, lane, K % BK);
    else
      oa.template issue<false>((const uint16_t*)c.ptr, c.left, lda, dst, sw, lane, BK);
    c.ptr += a_step;
    c.left -= a_step;
    if (++c.k == nk) {
      c.k = 0;
      if (++c.t < items) a_seek(c);
    }
  };
  auto copy_b = [&](Cursor& c, uint32_t buf) {
    const uint32_t dst = lds0 + B_BASE + buf * B_BYTES;
    if (k_ragged && c.k == nk - 1)
      ob.template issue<true>((const uint16_t*)c.ptr, c.left, ldb, dst, sw, lane, K % BK);
    else
      ob.template issue<false>((const uint16_t*)c.ptr, c.left, ldb, dst, sw, lane, BK);
    c.ptr += b_step;
    c.left -= b_step;
    if (++c.k == nk) {
      c.k = 0;
      if (++c.t < items) b_seek(c);
    }
  };

  // LDS byte offsets of this wave's fragment reads
  FragAddr<A_KC, OA::CH> fra;
  FragAddr<B_KC, OB::CH> frb;
  fra.init(wm0, lane);
  frb.init(wn0, lane);
  constexpr uint32_t A_TR4 = decltype(fra)::TR4, B_TR4 = decltype(frb)::TR4;

  f32x4 acc[FM][FN];
  u32x4 fa[KS][FM], fb[KS][FN];

  // memory phase: this wave's fragments of every slice of the step held in
  // A buffer abuf and B buffer bbuf
  auto mem = [&](uint32_t abuf, uint32_t bbuf) {
    const TG_LDS char* sa = lds + abuf * A_BYTES;
    const TG_LDS char* sb = lds + B_BASE + bbuf * B_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (A_KC) {
          fa[ks][i] = lds_read16(sa, fra.at(ks, i));
        } else {
          const u32x2 lo = lds_read_tr(sa, fra.at(ks, i)), hi = lds_read_tr(sa, fra.at(ks, i) + A_TR4);
          fa[ks][i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (B_KC) {
          fb[ks][j] = lds_read16(sb, frb.at(ks, j));
        } else {
          const u32x2 lo = lds_read_tr(sb, frb.at(ks, j)), hi = lds_read_tr(sb, frb.at(ks, j) + B_TR4);
          fb[ks][j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
    }
  };
  // MFMA phase: snake order over the blocks, so consecutive MFMAs share an
  // operand; the first step of an item starts from zero accumulators
  auto comp = [&](auto first) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          const int j = (i & 1) ? FN - 1 - jj : jj;
          if (decltype(first)::value && ks == 0)
            acc[i][j] = mfma16<In>(fb[ks][j], fa[ks][i], f32x4{});
          else
            acc[i][j] = mfma16<In>(fb[ks][j], fa[ks][i], acc[i][j]);
        }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Stores of item t's result (in acc).  A persistent launch (no epilogue,
  // N % 4 == 0, checked by the launcher) stores each finished item inside
  // the loop and every wave issues exactly ST vector stores -- a wave
  // outside C stores through an empty descriptor, which drops every access
  // -- because the counted waits allow exactly ST.  Otherwise the one item
  // is stored after the loop, with the epilogue and the element-wise path
  // for any N.
  const bool persistent = !EPI && (int64_t)gridDim.x < total;
  auto store_counted = [&](int32_t t) {
    const Item it = item_of(t);
    char* Cb = (char*)args.C + it.b * args.sC * (int64_t)sizeof(Out);
    const int64_t r0 = it.m0 + wm0, c0 = it.n0 + wn0;
    const bool in = r0 < M && c0 < N;
    store16_vec<Out, FM, FN>(in ? Cb + (r0 * ldc + c0) * (int64_t)sizeof(Out) : Cb,
                             in ? ((M - 1 - r0) * ldc + (N - c0)) * (int64_t)sizeof(Out) : 0, ldc, in ? N - c0 : 0,
                             lane, acc);
  };
  auto store_final = [&](int32_t t) {
    const Item it = item_of(t);
    char* Cb = (char*)args.C + it.b * args.sC * (int64_t)sizeof(Out);
    const int64_t r0 = it.m0 + wm0, c0 = it.n0 + wn0;
    if (r0 >= M || c0 >= N) return;
    if constexpr (EPI) epilogue16<Out, FM, FN>(args, Cb, ldc, M, N, r0, c0, lane, acc);
    if (N % 4 == 0 || it.n0 + BN <= N)
      store16_vec<Out, FM, FN>(Cb + (r0 * ldc + c0) * (int64_t)sizeof(Out),
                               ((M - 1 - r0) * ldc + (N - c0)) * (int64_t)sizeof(Out), ldc, N - c0, lane, acc);
    else
      store16_elem<Out, FM, FN>(Cb, ldc, M, N, r0, c0, lane, acc);
  };

  // Copy schedule (global step g; A in buffer g mod 3, B in buffer g mod 2):
  //  * prologue, group 0: A(0), B(0), A(1);
  //  * group 0's memory phase of step g: B(g + 1), into the buffer of step
  //    g - 1, which group 1 read in the previous phase; group 0 waits for it
  //    at the end of its MFMA phase, before the barrier after which it reads
  //    step g + 1;
  //  * group 1's memory phase of step g: A(g + 2), into the buffer of step
  //    g - 1; group 1 waits for A(g + 1) (its own copy of the previous
  //    phase, or group 0's prologue copy) at the end of this memory phase,
  //    before the barrier after which group 0 reads step g + 1.
  // Both groups move 32 KiB per step into LDS besides their 96 KiB of
  // fragment reads, so the two memory phases carry equal LDS traffic.
  Cursor cur{0, 0, nullptr, 0};
  if (grp == 0) {
    Cursor ca{0, 0, nullptr, 0};
    a_seek(ca);
    b_seek(cur);
    copy_a(ca, 0);
    copy_b(cur, 0);
    if (nsteps > 1) {
      copy_a(ca, 1);
      wait_vmcnt<PA, true>();  // A(0) and B(0) have landed; A(1) may not have
    } else {
      wait_vmcnt<0, true>();
    }
  } else {
    // group 1's cursor starts at A(2)
    cur.t = 2 / nk;
    cur.k = 2 - cur.t * nk;
    if (cur.t < items) a_seek(cur);
  }
  barrier();
  if (grp == 1) barrier();  // group 1 runs one phase behind

  // The K-step loop, compiled once per group and read/copy order (both are
  // uniform over a wave), so that each wave's loop carries only its own
  // copies and waits.
  auto run = [&](auto group, auto reads_first) {
    constexpr int G = decltype(group)::value;
    constexpr bool RF = decltype(reads_first)::value;
    int32_t kk = 0, t = 0;        // step within the item, item
    uint32_t abuf = 0, bbuf = 0;  // buffers of step g
    for (int32_t g = 0; g < nsteps; ++g) {
      fra.pin();
      frb.pin();
      oa.pin();
      ob.pin();
      // memory phase: this group's copies, the previous item's stores (after
      // the copies, so that the waits may leave them in flight) and the
      // fragments of step g -- fragments first in half of the waves (RF), so
      // that the copy burst (which holds a wave until the address unit takes
      // each copy) and the LDS reads proceed side by side
      const bool stored = !EPI && kk == 0 && g > 0;
      bool copied = false;
      if constexpr (RF) {
        mem(abuf, bbuf);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (G == 0) {
        if (g + 1 < nsteps) {
          copy_b(cur, bbuf ^ 1u);
          copied = true;
        }
      } else {
        if (g + 2 < nsteps) {
          copy_a(cur, abuf == 0 ? 2u : abuf - 1);
          copied = true;
        }
      }
      if constexpr (!EPI) {
        if (stored) store_counted(t - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!RF) mem(abuf, bbuf);
      if constexpr (G == 1) {
        // A(g + 1) has landed; A(g + 2) and the stores may still be in flight
        if (copied) {
          if (stored) wait_vmcnt<PA + ST, true>();
          else wait_vmcnt<PA, true>();
        } else {
          if (stored) wait_vmcnt<ST, true>();
          else wait_vmcnt<0, true>();
        }
      } else {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers
      }
      barrier();
      // the MFMA phase at a raised wave priority: when both waves of a SIMD
      // have an instruction ready, the MFMA goes first (measured 0.6-0.7%
      // faster on 8192^3, two boxes; raising the memory phase instead gained
      // nothing)
      __builtin_amdgcn_s_setprio(2);
      if (kk == 0)
        comp(std::true_type{});
      else
        comp(std::false_type{});
      __builtin_amdgcn_s_setprio(0);
      if constexpr (G == 0) {
        if (copied) {
          // B(g + 1) has landed; the stores issued after it may not have
          if (stored) wait_vmcnt<ST, false>();
          else wait_vmcnt<0, false>();
        }
      }
      if (G == 0 || g + 1 < nsteps) barrier();
      abuf = abuf == 2 ? 0u : abuf + 1;
      bbuf ^= 1u;
      if (++kk == nk) {
        kk = 0;
        ++t;
      }
    }
  };
  if (grp == 0) {
    if (sw < 2) run(std::integral_constant<int, 0>{}, std::false_type{});
    else run(std::integral_constant<int, 0>{}, std::true_type{});
  } else {
    if (sw < 2) run(std::integral_constant<int, 1>{}, std::false_type{});
    else run(std::integral_constant<int, 1>{}, std::true_type{});
  }
  if (persistent)
    store_counted(items - 1);
  else
    store_final(items - 1);
}

}  // namespace tg
