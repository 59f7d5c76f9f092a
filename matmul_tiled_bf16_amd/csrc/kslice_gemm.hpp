// kslice_gemm.hpp -- gfx950 GEMM/BMM for small, latency-bound products: the
// four waves of a work-group split one 64 x 64 output tile's K range.
//
// A product with few output tiles and a long K (1000^3: 256 tiles of 64 x 64,
// one per CU) is bound by the chain of K steps a tile walks: each step waits
// for copies that take a round trip to L2 or the Infinity Cache, and a ring
// of S stages hides at most S - 1 of them.  Splitting K four ways inside the
// work-group makes the chain four times shorter without a second launch or a
// reduction buffer ("Triton Optimization Reference", section 7: split-K and
// stream-K for tiles too few to fill the machine; here the split stays on one
// CU, so the partial sums meet in LDS):
//
//  * wave w walks K steps [w nk / 4, (w + 1) nk / 4) (32-deep steps) through
//    its own ring of STAGES LDS stages, copying its A and B tiles with
//    direct-to-LDS loads and reading them back like the tile kernel (same
//    swizzles, ds_read_b64_tr_b16 for M/N-contiguous operands); no other wave
//    touches its ring, so the K loop has no work-group barrier;
//  * each wave accumulates the whole 64 x 64 tile (2 x 2 blocks of
//    v_mfma_f32_32x32x16);
//  * the four partial tiles go to LDS (fp32) after one barrier, and wave w
//    sums 32 x 32 block w over the four, applies the epilogue and stores it.
#pragma once

#include "tile_gemm.hpp"

namespace tg {

template <typename In, typename Out, bool TA, bool TB, int STAGES>
__global__ void __launch_bounds__(256) kslice_gemm_kernel(GemmArgs args) {
  constexpr int BM = 64, BN = 64, BK = 32, NW = 4;
  constexpr bool A_KC = !TA, B_KC = TB;
  using DA = DmaOperand<A_KC, BM, BK, 1>;
  using DB = DmaOperand<B_KC, BN, BK, 1>;
  constexpr uint32_t A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2, STAGE = A_BYTES + B_BYTES;
  constexpr uint32_t RING = STAGES * STAGE;     // one wave's ring
  constexpr int PER_STEP = DA::INSTR + DB::INSTR;  // copy instructions per step (8)
  static_assert(STAGES >= 2 && (STAGES - 2) * PER_STEP < 64, "counted waits fit the vector-memory counter");
  static_assert(NW * RING >= NW * BM * BN * 4, "the partial tiles fit in the rings");

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;
  const uint32_t lds0 = (uint32_t)(size_t)lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb, ldc = args.ldc;
  const int64_t total = (int64_t)args.tiles_m * args.tiles_n * args.batch;
  const int64_t nk = (K + BK - 1) / BK;
  const int64_t s_begin = nk * wave / NW, s_end = nk * (wave + 1) / NW;
  const int32_t steps = (int32_t)(s_end - s_begin);

  DA da;
  DB db;
  da.init(0, lane, lda);
  db.init(0, lane, ldb);
  const uint32_t ring = lds0 + (uint32_t)wave * RING;
  const TG_LDS char* ring_p = lds + (uint32_t)wave * RING;

  for (int64_t w0 = blockIdx.x; w0 < total; w0 += gridDim.x) {
    int64_t b;
    int32_t pm, pn;
    work_coords<8>(w0, total, args.tiles_m, args.tiles_n, b, pm, pn);
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    const uint16_t* Ab = args.A + b * args.sA;
    const uint16_t* Bb = args.B + b * args.sB;
    // element offsets of the tile's step-0 origin and of the matrices' last
    // elements (+1): a copy's descriptor covers origin .. end of matrix, so
    // rows past M / N and K read zero
    const int64_t a_org = A_KC ? m0 * lda : m0, b_org = B_KC ? n0 * ldb : n0;
    const int64_t a_end = A_KC ? (M - 1) * lda + K : (K - 1) * lda + M;
    const int64_t b_end = B_KC ? (N - 1) * ldb + K : (K - 1) * ldb + N;
    const int64_t a_step = A_KC ? BK : BK * lda, b_step = B_KC ? BK : BK * ldb;

    auto issue = [&](int64_t s, uint32_t stage) __attribute__((always_inline)) {
      const int64_t ao = a_org + s * a_step, bo = b_org + s * b_step;
      const uint32_t dst = ring + stage * STAGE;
      if (s == nk - 1 && K % BK != 0) {
        da.template issue<true>(Ab + ao, (a_end - ao) * 2, dst, 0, K - s * BK);
        db.template issue<true>(Bb + bo, (b_end - bo) * 2, dst + A_BYTES, 0, K - s * BK);
      } else {
        da.template issue<false>(Ab + ao, (a_end - ao) * 2, dst, 0, K - s * BK);
        db.template issue<false>(Bb + bo, (b_end - bo) * 2, dst + A_BYTES, 0, K - s * BK);
      }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
      if (t < steps) issue(s_begin + t, (uint32_t)t);
    uint32_t stage = 0;
    for (int32_t t = 0; t < steps; ++t) {
      // step t's copies landed; the later ones issued so far may stay in flight
      const int32_t later = min(STAGES - 2, steps - 1 - t);
      if constexpr (STAGES >= 5) {
        if (later >= 3) wait_vmcnt<(STAGES >= 5 ? 3 : 0) * PER_STEP, true>();
      }
      if constexpr (STAGES >= 4) {
        if (later == 2) wait_vmcnt<2 * PER_STEP, true>();
      }
      if (later == 1) wait_vmcnt<PER_STEP, true>();
      else if (later == 0) wait_vmcnt<0, true>();
      const TG_LDS char* sa = ring_p + stage * STAGE;
      mma_stage<In, 2, 2, BK, A_KC, B_KC, DA::CH, DB::CH>(sa, sa + A_BYTES, 0, 0, lane, acc);
      // the stage read last is refilled STAGES - 1 steps ahead (its reads
      // are done: the MFMAs that consumed them have issued)
      const uint32_t prev = stage == 0 ? (uint32_t)(STAGES - 1) : stage - 1;
      if (t + STAGES - 1 < steps) issue(s_begin + t + STAGES - 1, prev);
      stage = stage == (uint32_t)(STAGES - 1) ? 0u : stage + 1;
    }

    // partial tiles through LDS: wave w's block (i, j) at slot (w, i, j),
    // register r of lane l at (r * 64 + l) * 4 -- then wave w sums block
    // (w >> 1, w & 1) over the four waves
    wait_vmcnt<0, true>();
    block_barrier();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          TG_LDS float* dst = (TG_LDS float*)(lds + (uint32_t)(((wave * 4 + i * 2 + j) * 16 + r) * 256 + lane * 16));
          *(TG_LDS f32x4*)dst = f32x4{acc[i][j][r], acc[i][j][r + 1], acc[i][j][r + 2], acc[i][j][r + 3]};
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's partials are in LDS
    block_barrier();
    const int bi = wave >> 1, bj = wave & 1;
    f32x16 sum[1][1];
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[0][0][r] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const f32x4 v =
            *(const TG_LDS f32x4*)(lds + (uint32_t)(((w * 4 + bi * 2 + bj) * 16 + r) * 256 + lane * 16));
        sum[0][0][r] += v[0];
        sum[0][0][r + 1] += v[1];
        sum[0][0][r + 2] += v[2];
        sum[0][0][r + 3] += v[3];
      }

    char* Cb = (char*)args.C + b * args.sC * (int64_t)sizeof(Out);
    const int64_t r0 = m0 + bi * 32, c0 = n0 + bj * 32;
    if (args.epi) epilogue_acc<Out, 1, 1>(args, Cb, ldc, M, N, r0, c0, lane, sum);
    if (r0 < M && c0 < N) {
      if (N % 4 == 0 || c0 + 32 <= N)
        store_tile_vec<Out, 1, 1>(Cb + (r0 * ldc + c0) * (int64_t)sizeof(Out),
                                  ((M - 1 - r0) * ldc + (N - c0)) * (int64_t)sizeof(Out), ldc, N - c0, lane, sum);
      else
        store_tile<Out, 1, 1>(Cb, ldc, M, N, r0, c0, lane, sum);
    }
    if (w0 + gridDim.x < total) block_barrier();  // the next item's copies refill the rings
  }
}

}  // namespace tg
