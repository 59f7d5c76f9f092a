// skinny_gemm.hpp -- gfx950 kernel for tall-thin products: M <= 32 rows of C,
// A (M x K) and B (stored N x K) both contiguous along K.
//
// Such a product moves ~2*N*K bytes of B for only 2*M*N*K flops, so it is
// bound by HBM, not by the matrix cores ("Optimize Triton Block Parameters",
// Step 1 classification; Performance requirements: a memory-bound kernel
// wants many loads in flight, a small-M shape wants a small BLOCK_M).  The
// kernel therefore streams every byte of B exactly once, straight from global
// memory into v_mfma_f32_16x16x32 operand registers:
//   * lane (j = lane & 15, g = lane >> 4) of a wave loads 16 bytes -- 8
//     consecutive k -- of row j of stored B, which is exactly the B operand
//     layout of the 16x16x32 MFMA; A rows are read the same way (they stay
//     in L2, every work-group reads all of A);
//   * a work-group owns 16*NBLK columns of C; its WAVES waves split K into
//     contiguous slices and each keeps UNROLL k-blocks of loads in flight;
//   * the per-wave fp32 partial tiles are summed through LDS in a fixed wave
//     order (deterministic), then rounded and stored.
// No LDS staging of B is needed: both operands are K-contiguous, so the
// layout the loads produce is already the layout the MFMA consumes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace tg {

// MB: 16-row blocks of C (M <= 16*MB); NBLK: 16-column blocks per
// work-group; WAVES waves split K; UNROLL 32-deep K blocks per load batch.
template <typename In, typename Out, int MB, int NBLK, int WAVES, int UNROLL>
__global__ void __launch_bounds__(WAVES * 64) skinny_gemm_kernel(GemmArgs args) {
  extern __shared__ __attribute__((aligned(16))) char tg_smem[];
  float* red = (float*)tg_smem;  // [WAVES][MB][NBLK][64 lanes][4]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lj = lane & 15, lg = lane >> 4;
  const int64_t M = args.M, N = args.N, K = args.K;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * NBLK);

  // K slice of this wave, in whole 32-element MFMA blocks
  const int64_t kb = (K + 31) / 32;
  const int64_t per = (kb + WAVES - 1) / WAVES;
  const int64_t k_begin = min((int64_t)wave * per * 32, K);
  const int64_t k_end = min((int64_t)(wave + 1) * per * 32, K);

  for (int64_t b = blockIdx.y; b < args.batch; b += gridDim.y) {
    const uint16_t* Ab = args.A + b * args.sA;
    const uint16_t* Bb = args.B + b * args.sB;
    const uint16_t* arow[MB];
    const uint16_t* brow[NBLK];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int64_t r = i * 16 + lj;
      arow[i] = Ab + (r < M ? r : M - 1) * args.lda + lg * 8;
    }
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
      const int64_t r = n0 + j * 16 + lj;
      brow[j] = Bb + (r < N ? r : N - 1) * args.ldb + lg * 8;
    }

    f32x4 acc[MB][NBLK];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBLK; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    int64_t k = k_begin;
    // steady state: UNROLL whole 32-k blocks, no masks
    for (; k + 32 * UNROLL <= k_end; k += 32 * UNROLL) {
      u32x4 av[UNROLL][MB], bv[UNROLL][NBLK];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j) bv[u][j] = *(const u32x4*)(brow[j] + k + u * 32);
#pragma unroll
        for (int i = 0; i < MB; ++i) av[u][i] = *(const u32x4*)(arow[i] + k + u * 32);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NBLK; ++j) acc[i][j] = mfma16<In>(av[u][i], bv[u][j], acc[i][j]);
    }
    // remaining 32-k blocks of the slice; 8-element chunks at or past k_end are zero
    for (; k < k_end; k += 32) {
      const bool ok = k + lg * 8 < k_end;
      u32x4 av[MB], bv[NBLK];
#pragma unroll
      for (int j = 0; j < NBLK; ++j) bv[j] = ok ? *(const u32x4*)(brow[j] + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < MB; ++i) av[i] = ok ? *(const u32x4*)(arow[i] + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBLK; ++j) acc[i][j] = mfma16<In>(av[i], bv[j], acc[i][j]);
    }

    // cross-wave reduction in a fixed order
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBLK; ++j)
        *(f32x4*)(red + (((wave * MB + i) * NBLK + j) * 64 + lane) * 4) = acc[i][j];
    __syncthreads();
    constexpr int OUTS = MB * 16 * NBLK * 16;
    Out* Cb = (Out*)args.C + b * args.sC;
    for (int e = tid; e < OUTS; e += WAVES * 64) {
      const int row = e / (NBLK * 16), col = e % (NBLK * 16);
      const int i = row >> 4, rr = row & 15, j = col >> 4;
      const int src_lane = (rr >> 2) * 16 + (col & 15), r = rr & 3;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) s += red[(((w * MB + i) * NBLK + j) * 64 + src_lane) * 4 + r];
      const int64_t gc = n0 + col;
      if (row < M && gc < N) store_out<Out>(Cb, row * args.ldc + gc, s);
    }
    __syncthreads();
  }
}

}  // namespace tg
