// skinny_gemm.hpp -- gfx950 kernel for tall-thin products: M <= 32 rows of C,
// A (M x K) and B (stored N x K) both contiguous along K.
//
// Such a product moves ~2*N*K bytes of B for only 2*M*N*K flops, so it is
// bound by HBM, not by the matrix cores ("Optimize Triton Block Parameters",
// Step 1 classification; Performance requirements: a memory-bound kernel
// wants many loads in flight, a small-M shape wants a small BLOCK_M).  The
// kernel streams every byte of B once and spends its effort on the access
// pattern the memory system sees (each point below was measured on MI355X):
//   * a work-group owns 16*NB rows of B (16*NB columns of C) and walks K in
//     stages of SK elements; A's rows for the same stage come along, so every
//     A byte fetched from L2 serves NB row-blocks of B;
//   * A and B move into an LDS ring of S stage buffers by direct-to-LDS
//     buffer loads whose 64 lanes cover 1 KiB as whole 2*SK-byte row
//     segments (loads shaped like an MFMA operand, 16 rows x 64 bytes, ran
//     ~40% slower); B's loads are non-temporal, it is read once;
//   * work-groups run in lock-step, so each one starts its K walk at a
//     different stage -- otherwise all of them hit the same lines of A and
//     the same HBM channels of B at once;
//   * one barrier per stage: a wave waits for its own loads of stage t, the
//     barrier publishes the whole stage, and the loads of stage t+S-1 go into
//     the buffer every wave finished reading one step earlier;
//   * v_mfma_f32_16x16x32 takes its operands (row j, 8 consecutive k per
//     lane) from LDS through an XOR swizzle of the 16-byte chunks that keeps
//     16 rows on distinct banks; each wave owns fixed (k-block, row-block)
//     pairs of every stage and the per-wave fp32 partials are summed through
//     LDS in a fixed wave order (deterministic), then rounded and stored.
// Chunks past K, rows past N and rows of A past M get a buffer offset beyond
// the descriptor's size and read zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace tg {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t skinny_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// 16 bytes per lane straight into LDS at dst + 16*lane (dst is wave-uniform)
template <int AUX>
__device__ __forceinline__ void skinny_dma(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                           __attribute__((address_space(3))) void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (int)off, 0, 0, AUX);
}

// Wait until at most N of this wave's vector loads are outstanding and all of
// its LDS reads have returned.  The LDS part matters: the buffer refilled
// right after the next barrier is the one read in the step before it, and a
// refill that reads out of range (past K) is answered with zeros at once,
// without a trip to memory -- so every wave's reads of that buffer must be
// complete before any wave may pass the barrier.
template <int N>
__device__ __forceinline__ void skinny_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0)
}

// A work-group barrier that orders memory operations for the compiler only;
// each wave has already waited for what the others must see.
__device__ __forceinline__ void skinny_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MB: 16-row blocks of A/C (M <= 16*MB); NB: 16-row blocks of B per
// work-group; WAVES waves; S stage buffers; SK k-elements per stage.
template <typename In, typename Out, int MB, int NB, int WAVES, int S, int SK>
__global__ void __launch_bounds__(WAVES * 64) skinny_gemm_kernel(GemmArgs args) {
  static_assert(S >= 3 && S <= 8, "3 to 8 stage buffers");
  static_assert(SK == 128 || SK == 256, "stage depth");
  constexpr int ROWB = SK * 2;               // bytes of one row in a stage
  constexpr int CH = ROWB / 16;              // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;           // rows per load instruction
  constexpr int BROWS = 16 * NB, AROWS = 16 * MB;
  constexpr int BI = BROWS / RPI, AI = AROWS / RPI;
  static_assert(BI % WAVES == 0 && AI % WAVES == 0, "loads split evenly over the waves");
  constexpr int PWB = BI / WAVES, PWA = AI / WAVES;  // load instructions per wave per stage
  constexpr int PW = PWB + PWA;
  constexpr int B_BYTES = BROWS * ROWB;
  constexpr int SLOT = (BROWS + AROWS) * ROWB;
  constexpr int KB = SK / 32;                // MFMA k-blocks per stage
  constexpr int IPW = KB * NB / WAVES;       // (k-block, row-block) items per wave
  static_assert((KB * NB) % WAVES == 0 && IPW >= 1, "MFMA items split evenly over the waves");
  constexpr uint32_t kOff = 0x80000000u;     // beyond any descriptor size: reads zero
  using LdsPtr = __attribute__((address_space(3))) char*;

  // one array per ring buffer: the compiler tracks outstanding direct-to-LDS
  // loads per array, so its own waits before reading a buffer cover only the
  // loads into that buffer
  __shared__ __attribute__((aligned(1024))) char sb0[SLOT];
  __shared__ __attribute__((aligned(1024))) char sb1[SLOT];
  __shared__ __attribute__((aligned(1024))) char sb2[SLOT];
  __shared__ __attribute__((aligned(1024))) char sb3[S > 3 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) char sb4[S > 4 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) char sb5[S > 5 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) char sb6[S > 6 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) char sb7[S > 7 ? SLOT : 16];
  auto slot = [&](int s) -> LdsPtr {
    switch (s) {
      case 0: return (LdsPtr)sb0;
      case 1: return (LdsPtr)sb1;
      case 2: return (LdsPtr)sb2;
      case 3: return (LdsPtr)sb3;
      case 4: return (LdsPtr)sb4;
      case 5: return (LdsPtr)sb5;
      case 6: return (LdsPtr)sb6;
      default: return (LdsPtr)sb7;
    }
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lj = lane & 15, lg = lane >> 4;
  const int64_t M = args.M, N = args.N, K = args.K;
  const int64_t n0 = (int64_t)blockIdx.x * BROWS;
  const int64_t rows_b = min((int64_t)BROWS, N - n0);

  // stages: index idx = 0 .. nst-1 walks stage (idx + rot) mod nst
  const int nst = (int)((K + SK - 1) / SK);
  const int rounds = (nst + S - 1) / S;
  const int rot = (int)(blockIdx.x % (unsigned)nst);

  // this wave's load instructions: its p-th B load is instruction
  // t = wave*PWB + p of B, filling rows t*RPI .. of the buffer's B part; its
  // p-th A load likewise in the A part.  A lane lands at chunk lane%CH of its
  // row and fetches the chunk the swizzle puts there.
  uint32_t ld_off[PW], ld_chunk[PW];
  bool ld_ok[PW];
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    const bool is_b = p < PWB;
    const int t = is_b ? wave * PWB + p : wave * PWA + (p - PWB);
    const int row = t * RPI + lane / CH;
    const int c = (lane % CH) ^ (row & 15);
    ld_ok[p] = is_b ? row < rows_b : row < M;
    ld_off[p] = (uint32_t)(row * (is_b ? args.ldb : args.lda) * 2 + c * 16);
    ld_chunk[p] = c;
  }
  // this wave's MFMA items: item it = wave*IPW + u is k-block it / NB of
  // row-block it % NB; lane (j, g) reads row j, chunk kb*4 + g
  uint32_t rd_b[IPW], rd_a[IPW][MB];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int it = wave * IPW + u, kb = it / NB, rb = it % NB;
    const uint32_t chunk = (uint32_t)(((kb * 4 + lg) ^ lj) * 16);
    rd_b[u] = (rb * 16 + lj) * ROWB + chunk;
#pragma unroll
    for (int i = 0; i < MB; ++i) rd_a[u][i] = B_BYTES + (i * 16 + lj) * ROWB + chunk;
  }

  for (int64_t b = blockIdx.y; b < args.batch; b += gridDim.y) {
    const uint16_t* Ab = args.A + b * args.sA;
    const uint16_t* Bb = args.B + b * args.sB + n0 * args.ldb;
    const __amdgpu_buffer_rsrc_t rsa = skinny_rsrc(Ab, ((M - 1) * args.lda + K) * 2);
    const __amdgpu_buffer_rsrc_t rsb = skinny_rsrc(Bb, ((rows_b - 1) * args.ldb + K) * 2);

    auto dma = [&](int s, int idx) {
      const bool live = idx < nst;
      int st = idx + rot;
      st = st >= nst ? st - nst : st;
#pragma unroll
      for (int p = 0; p < PW; ++p) {
        const bool ok = live && ld_ok[p] && (int64_t)st * SK + ld_chunk[p] * 8 < K;
        const uint32_t off = ok ? ld_off[p] + (uint32_t)st * ROWB : kOff;
        if (p < PWB)  // B: read once, non-temporal
          skinny_dma<2>(rsb, off, slot(s) + (wave * PWB + p) * 1024);
        else
          skinny_dma<0>(rsa, off, slot(s) + B_BYTES + (wave * PWA + p - PWB) * 1024);
      }
    };

    f32x4 acc[IPW][MB];
#pragma unroll
    for (int u = 0; u < IPW; ++u)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int s) {
      const LdsPtr base = slot(s);
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const u32x4 bv = *(const __attribute__((address_space(3))) u32x4*)(base + rd_b[u]);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const u32x4 av = *(const __attribute__((address_space(3))) u32x4*)(base + rd_a[u][i]);
          acc[u][i] = mfma16<In>(av, bv, acc[u][i]);
        }
      }
    };

    // prologue: S-1 stages in flight
#pragma unroll
    for (int s = 0; s < S - 1; ++s) dma(s, s);
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int idx = r * S + s;
        skinny_wait_vmcnt<(S - 2) * PW>();  // own loads of stage idx landed, own reads done
        skinny_barrier();                   // ... everyone's: buffer s-1 is free
        dma((s + S - 1) % S, idx + S - 1);
        compute(s);
      }
    }

    // cross-wave reduction in a fixed order, through buffer 0 (after the last
    // refills, which read zero, have landed): partial of item u of wave w is
    // red[w][u]; the output block of row-block rb sums the items with that rb
    skinny_wait_vmcnt<0>();
    __syncthreads();
    float* red = (float*)sb0;  // [WAVES][IPW][MB][64 lanes][4]
    static_assert(WAVES * IPW * MB * 64 * 16 <= SLOT, "reduction fits in buffer 0");
#pragma unroll
    for (int u = 0; u < IPW; ++u)
#pragma unroll
      for (int i = 0; i < MB; ++i) *(f32x4*)(red + (((wave * IPW + u) * MB + i) * 64 + lane) * 4) = acc[u][i];
    __syncthreads();
    constexpr int OUTS = AROWS * BROWS;
    Out* Cb = (Out*)args.C + b * args.sC;
    for (int e = tid; e < OUTS; e += WAVES * 64) {
      const int row = e / BROWS, col = e % BROWS;
      const int i = row >> 4, rr = row & 15, rb = col >> 4;
      const int src_lane = (rr >> 2) * 16 + (col & 15), q = rr & 3;
      float sum = 0.f;
      // items it = w*IPW + u with it % NB == rb, in increasing it (fixed order)
#pragma unroll
      for (int it = rb; it < KB * NB; it += NB) sum += red[((it * MB + i) * 64 + src_lane) * 4 + q];
      const int64_t gc = n0 + col;
      if (row < M && gc < N) {
        if (args.epi) {  // alpha * sum + beta * C + bias, as epilogue_acc
          sum *= args.alpha;
          if (args.beta != 0.f) sum = __builtin_fmaf(args.beta, load_out<Out>(Cb, row * args.ldc + gc), sum);
          if (args.bias) sum += load_out<Out>(args.bias, gc);
        }
        store_out<Out>(Cb, row * args.ldc + gc, sum);
      }
    }
    __syncthreads();
  }
}

}  // namespace tg
