// common.hpp -- pieces shared by the gfx950 GEMM kernels: MFMA wrappers, LDS
// layout (swizzle) and fragment reads, tile scheduling and the epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

#define TG_LDS __attribute__((address_space(3)))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;  // batch strides, elements
  int64_t batch;
  int32_t tiles_m, tiles_n;
  int32_t rotate_k;  // nonzero: each work-group starts its walk over K at a different step
  int32_t persist;   // nonzero: the next item's first stages are issued before this item's stores
  // epilogue: C = alpha * acc + beta * C + bias[col] when epi != 0 (C is
  // read only if beta != 0; bias, of the output type, may be null)
  int32_t epi;
  float alpha, beta;
  const void* bias;
  int32_t stream_c;  // nonzero: LDS-staged C stores are non-temporal
  int32_t span;      // panel kernel: column tiles per run of a work-group
  int32_t nt_ab;     // tile kernel: bit 0 (1): A, bit 1 (2): B is read by one tile only -- non-temporal loads
};

using KernelFn = void (*)(GemmArgs);

// A grouped launch: up to kGroupMax independent products of different shapes
// (same types and transposes) in one grid.  Work items are numbered problem
// by problem; problem i owns items [first, first + tiles), its tiles in
// column-major order.  The table travels in the kernel-argument segment, so the launch
// needs no device memory of its own.
constexpr int kGroupMax = 32;
struct GroupProblem {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t first;  // first work item of this problem
};
struct GroupArgs {
  GemmArgs g;      // shared launch fields (rotate_k and persist are 0)
  int32_t count;   // problems in the table, 1 .. kGroupMax
  int32_t total;   // work items of all problems
  GroupProblem p[kGroupMax];
};
using GroupFn = void (*)(GroupArgs);

// ---------------------------------------------------------------- MFMA ---
// v_mfma_f32_32x32x16: for D = X Y, lane l supplies row (l & 31) of X and
// column (l & 31) of Y, each as 8 consecutive k starting at 8*(l >> 5);
// register r of the result holds D[8*(r>>2) + 4*(l>>5) + (r&3)][l & 31].
// The kernels pass the B fragment as X and the A fragment as Y, so they
// accumulate C^T: register r of lane l holds C[l & 31][8*(r>>2) + 4*(l>>5) +
// (r&3)] -- four consecutive columns of one row per group of 4 registers,
// which the epilogue writes as one 8- or 16-byte store.
template <typename In>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<__bf16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<_Float16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                 0, 0, 0);
}

// v_mfma_f32_16x16x32: lane l supplies row/column (l & 15) as 8 consecutive k
// starting at 8*(l >> 4); register r holds C[4*(l>>4) + r][l & 15].
template <typename In>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16<__bf16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<_Float16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
}

// ------------------------------------------------------------ epilogue ---
template <typename Out>
__device__ __forceinline__ void store_out(void* C, int64_t off, float v);
template <>
__device__ __forceinline__ void store_out<float>(void* C, int64_t off, float v) {
  static_cast<float*>(C)[off] = v;
}
template <>
__device__ __forceinline__ void store_out<__bf16>(void* C, int64_t off, float v) {
  static_cast<__bf16*>(C)[off] = (__bf16)v;  // v_cvt_pk_bf16_f32: nearest, ties to even
}
template <>
__device__ __forceinline__ void store_out<_Float16>(void* C, int64_t off, float v) {
  static_cast<_Float16*>(C)[off] = (_Float16)v;
}

template <typename Out>
__device__ __forceinline__ float load_out(const void* C, int64_t off) {
  return (float)static_cast<const Out*>(C)[off];
}

// The epilogue on a wave's FM x FN accumulator blocks (acc holds C^T, see
// mfma32), in fp32 before any store path: acc = alpha*acc + beta*C + bias.
// Rows/columns past M/N are not read; their values are never stored.
template <typename Out, int FM, int FN>
__device__ __forceinline__ void epilogue_acc(const GemmArgs& args, const void* Cb, int64_t ldc, int64_t M, int64_t N,
                                             int64_t r0, int64_t c0, int lane, f32x16 (&acc)[FM][FN]) {
  const int li = lane & 31, lg = lane >> 5;
  const float alpha = args.alpha, beta = args.beta;
  const bool use_c = beta != 0.f, use_bias = args.bias != nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = r0 + i * 32 + li;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t col = c0 + j * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        float v = alpha * acc[i][j][r];
        if (row < M && col < N) {
          if (use_c) v = __builtin_fmaf(beta, load_out<Out>(Cb, row * ldc + col), v);
          if (use_bias) v += load_out<Out>(args.bias, col);
        }
        acc[i][j][r] = v;
      }
    }
  }
}

// --------------------------------------------------------- LDS helpers ---
__device__ __forceinline__ u32x4 lds_read16(const TG_LDS char* base, uint32_t off) {
  return *(const TG_LDS u32x4*)(base + off);
}
__device__ __forceinline__ void lds_write16(TG_LDS char* base, uint32_t off, u32x4 v) {
  *(TG_LDS u32x4*)(base + off) = v;
}
// Transposing read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives element (i & 3) of the 8-byte words addressed by lanes (i >> 2),
// 4 + (i >> 2), 8 + (i >> 2) and 12 + (i >> 2).  So if lane s addresses row
// r0 + (s >> 2), columns c0 + 4*(s & 3) .. +3 of a row-major 16-bit tile,
// lane i ends up with column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ u32x2 lds_read_tr(const TG_LDS char* base, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS i16x4*)(base + off)));
}

// LDS swizzle, in 16-byte units.  A tile row is CH units long.  gfx950's
// LDS serves 256 bytes (64 banks) per clock, i.e. 16 lanes of a
// ds_read_b128 or of a ds_read_b64_tr_b16 group pair per clock.
//  * K-contiguous tiles (rows along M/N, CH = BK/8): a fragment read puts 16
//    consecutive rows at one K offset in the same clock.  With W = 16/CH rows
//    per 256-byte window, flipping the unit index by (row / W) makes those 16
//    rows land on 16 distinct 16-byte slots.
//  * M/N-contiguous tiles (rows along K): one transposing read has four rows
//    at the same column offset per 16 lanes; flipping by a per-row pattern
//    with distinct bits 1-2 and distinct bits 2-3 keeps those rows apart in
//    both 128-byte and 256-byte windows.
template <bool KCONTIG, int CH>
__device__ __forceinline__ uint32_t swz_unit(uint32_t row) {
  if constexpr (KCONTIG) {
    static_assert(CH == 4 || CH == 8 || CH == 16, "K-contiguous rows of 32, 64 or 128 elements");
    constexpr uint32_t shift = CH == 4 ? 2 : CH == 8 ? 1 : 0;
    return (row >> shift) & (uint32_t)(CH - 1);
  } else {
    const uint32_t r = row & 3u;
    return ((r << 1) | ((r & 1u) << 3)) & (uint32_t)(CH - 1);
  }
}

template <bool KCONTIG, int CH>
__device__ __forceinline__ uint32_t swz_off(uint32_t row, uint32_t col) {
  return row * (CH * 16u) + (((col >> 3) ^ swz_unit<KCONTIG, CH>(row)) << 4) + ((col & 7u) << 1);
}

// ------------------------------------------------------ tile scheduling ---
// The hardware hands consecutive work-group ids to the 8 XCDs in turn.  Give
// XCD x the contiguous id range [x*G/8, (x+1)*G/8) instead, then decode that
// id in bands of GROUP_M tile rows so that work-groups running together on one
// XCD share A rows and B columns in that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int32_t bid, int32_t tiles_m, int32_t tiles_n, int32_t& pm,
                                            int32_t& pn) {
  const int32_t G = tiles_m * tiles_n;
  const int32_t per = G >> 3, rem = G & 7;
  const int32_t x = bid & 7, local = bid >> 3;
  const int32_t id = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
  const int32_t band = GROUP_M * tiles_n;
  const int32_t bidx = id / band;
  const int32_t first_m = bidx * GROUP_M;
  const int32_t gsz = min(tiles_m - first_m, GROUP_M);
  const int32_t in_band = id - bidx * band;
  pm = first_m + in_band % gsz;
  pn = in_band / gsz;
}

// Flat work index -> (matrix of the batch, tile row, tile column).  Work
// item w0 is assumed to run on XCD w0 mod 8 (the dispatcher deals
// consecutive work-groups round-robin over the XCDs, and a grid that loops
// over work items strides by a multiple of 8).  Each XCD gets one contiguous
// run of the (batch, tile) sequence, so a matrix's tiles -- which share that
// matrix's A and B -- meet in one XCD's L2 instead of all eight; inside a
// matrix, tiles go in bands of GROUP_M tile rows as in tile_coords.
template <int GROUP_M>
__device__ __forceinline__ void work_coords(int64_t w0, int64_t total, int32_t tiles_m, int32_t tiles_n,
                                            int64_t& b, int32_t& pm, int32_t& pn) {
  const int64_t per = total >> 3, rem = total & 7;
  const int64_t x = w0 & 7, local = w0 >> 3;
  const int64_t id = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
  const int64_t G = (int64_t)tiles_m * tiles_n;
  b = id / G;
  const int32_t t = (int32_t)(id - b * G);
  const int32_t band = GROUP_M * tiles_n;
  const int32_t bidx = t / band;
  const int32_t first_m = bidx * GROUP_M;
  const int32_t gsz = min(tiles_m - first_m, GROUP_M);
  const int32_t in_band = t - bidx * band;
  pm = first_m + in_band % gsz;
  pn = in_band / gsz;
}

// ---------------------------------------------------- one LDS stage of MMA ---
// A wave owns FM x FN blocks of 32x32 starting at (wm0, wn0) inside the tile.
// K-contiguous operands are read with ds_read_b128 (8 consecutive k of one
// row); M/N-contiguous ones with two transposing reads (4 k each), which
// give the same k-to-register assignment.
template <typename In, int FM, int FN, int BK, bool A_KC, bool B_KC, int A_CH, int B_CH>
__device__ __forceinline__ void mma_stage(const TG_LDS char* sa, const TG_LDS char* sb, int wm0, int wn0, int lane,
                                          f32x16 (&acc)[FM][FN]) {
  const int li = lane & 31, lg = lane >> 5;
  const int trh = lane >> 4, trs = lane & 15;
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    u32x4 af[FM], bf[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm0 + i * 32;
      if constexpr (A_KC) {
        af[i] = lds_read16(sa, swz_off<true, A_CH>(rb + li, ks * 16 + lg * 8));
      } else {
        const int col = rb + 16 * (trh & 1) + 4 * (trs & 3);
        const int kr = ks * 16 + 8 * (trh >> 1) + (trs >> 2);
        const u32x2 lo = lds_read_tr(sa, swz_off<false, A_CH>(kr, col));
        const u32x2 hi = lds_read_tr(sa, swz_off<false, A_CH>(kr + 4, col));
        af[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cb = wn0 + j * 32;
      if constexpr (B_KC) {
        bf[j] = lds_read16(sb, swz_off<true, B_CH>(cb + li, ks * 16 + lg * 8));
      } else {
        const int col = cb + 16 * (trh & 1) + 4 * (trs & 3);
        const int kr = ks * 16 + 8 * (trh >> 1) + (trs >> 2);
        const u32x2 lo = lds_read_tr(sb, swz_off<false, B_CH>(kr, col));
        const u32x2 hi = lds_read_tr(sb, swz_off<false, B_CH>(kr + 4, col));
        bf[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<In>(bf[j], af[i], acc[i][j]);
  }
}

// Element-wise masked store of a wave's FM x FN 32x32 blocks of C (any
// alignment; rows/cols past M/N dropped).  acc[i][j] holds C^T (see above).
template <typename Out, int FM, int FN>
__device__ __forceinline__ void store_tile(void* Cb, int64_t ldc, int64_t M, int64_t N, int64_t r0, int64_t c0,
                                           int lane, const f32x16 (&acc)[FM][FN]) {
  const int li = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = r0 + i * 32 + li;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t col = c0 + j * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (row < M && col < N) store_out<Out>(Cb, row * ldc + col, acc[i][j][r]);
      }
    }
  }
}

}  // namespace tg
