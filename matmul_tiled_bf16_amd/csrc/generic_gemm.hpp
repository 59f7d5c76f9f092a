// generic_gemm.hpp -- gfx950 tiled GEMM/BMM for any alignment and leading
// dimension: the same LDS layout and MFMA core as the vector kernel, but each
// 16-byte LDS unit is gathered element by element with bounds checks (zero
// outside the matrix), staged in registers and written with ds_write_b128.
// It serves operands whose base, leading dimension or contiguous extent is
// not a multiple of 8 elements ("Triton Optimization Reference", section 6:
// wide transactions only where alignment is known).
#pragma once

#include "common.hpp"

namespace tg {

template <bool KC, int MN_T, int BK, int NT>
struct GatherOperand {
  static constexpr int CH = KC ? BK / 8 : MN_T / 8;
  static constexpr int UNITS = MN_T * BK / 8;
  static constexpr int PER_THREAD = UNITS / NT;
  static_assert(UNITS % NT == 0, "tile must split evenly over the work-group");

  u32x4 reg[PER_THREAD];

  // Unit q of the tile: LDS row q / CH, logical 16-byte unit q % CH.
  __device__ __forceinline__ void load(const uint16_t* X, int64_t ld, int64_t mn0, int64_t mn, int64_t k0,
                                       int64_t K, int tid) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int q = tid + u * NT;
      const int row = q / CH, unit = q % CH;
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 2 * p + h;
          const int64_t kk = KC ? k0 + unit * 8 + e : k0 + row;
          const int64_t mm = KC ? mn0 + row : mn0 + unit * 8 + e;
          half[h] = (kk < K && mm < mn) ? (uint32_t)X[KC ? mm * ld + kk : kk * ld + mm] : 0u;
        }
        w[p] = half[0] | (half[1] << 16);
      }
      reg[u] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }

  __device__ __forceinline__ void store(TG_LDS char* tile, int tid) const {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int q = tid + u * NT;
      const int row = q / CH, unit = q % CH;
      lds_write16(tile, swz_off<KC, CH>(row, unit * 8), reg[u]);
    }
  }
};

template <typename In, typename Out, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB>
__global__ void __launch_bounds__(WM * WN * 64) generic_gemm_kernel(GemmArgs args) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr bool A_KC = !TA, B_KC = TB;
  using GA = GatherOperand<A_KC, BM, BK, NT>;
  using GB = GatherOperand<B_KC, BN, BK, NT>;
  constexpr uint32_t A_BYTES = BM * BK * 2, STAGE = A_BYTES + BK * BN * 2;

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
  const int64_t M = args.M, N = args.N, K = args.K;
  const int64_t nk = (K + BK - 1) / BK;

  GA ga;
  GB gb;
  const int64_t total = (int64_t)args.tiles_m * args.tiles_n * args.batch;
  for (int64_t w0 = blockIdx.x; w0 < total; w0 += gridDim.x) {
    int64_t b;
    int32_t pm, pn;
    work_coords<8>(w0, total, args.tiles_m, args.tiles_n, b, pm, pn);
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    const uint16_t* Ab = args.A + b * args.sA;
    const uint16_t* Bb = args.B + b * args.sB;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
      ga.load(Ab, args.lda, m0, M, 0, K, tid);
      gb.load(Bb, args.ldb, n0, N, 0, K, tid);
      ga.store(lds, tid);
      gb.store(lds + A_BYTES, tid);
      __syncthreads();
    }
    for (int64_t kt = 0; kt < nk; ++kt) {
      const uint32_t st = (uint32_t)(kt & 1);
      const bool more = kt + 1 < nk;
      if (more) {
        ga.load(Ab, args.lda, m0, M, (kt + 1) * BK, K, tid);
        gb.load(Bb, args.ldb, n0, N, (kt + 1) * BK, K, tid);
      }
      const TG_LDS char* sa = lds + st * STAGE;
      mma_stage<In, FM, FN, BK, A_KC, B_KC, GA::CH, GB::CH>(sa, sa + A_BYTES, wm0, wn0, lane, acc);
      if (more) {
        TG_LDS char* nx = lds + (st ^ 1u) * STAGE;
        ga.store(nx, tid);
        gb.store(nx + A_BYTES, tid);
      }
      __syncthreads();
    }
    void* Cb = (char*)args.C + b * args.sC * (int64_t)sizeof(Out);
    if (args.epi) epilogue_acc<Out, FM, FN>(args, Cb, args.ldc, M, N, m0 + wm0, n0 + wn0, lane, acc);
    store_tile<Out, FM, FN>(Cb, args.ldc, M, N, m0 + wm0, n0 + wn0, lane, acc);
  }
}

}  // namespace tg
