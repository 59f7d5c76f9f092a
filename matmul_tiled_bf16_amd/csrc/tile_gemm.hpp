// tile_gemm.hpp -- gfx950 tiled GEMM/BMM with direct HBM->LDS loads.
//
// One work-group computes a BM x BN tile of C[b] = op(A[b]) op(B[b]); K is
// walked in BK-deep steps through a ring of STAGES LDS buffers.
//
//  * Staging: every K step's A tile (BM x BK) and B tile (BK x BN) is copied
//    by buffer_load_dwordx4 ... lds, which writes each lane's 16 bytes
//    straight into LDS (lane t of one instruction lands at base + 16 t) with
//    no trip through registers.  The LDS layout is swizzled by choosing which
//    16-byte source unit each lane fetches; lanes sharing a row still read
//    that row's bytes, so the global side stays coalesced along each
//    operand's contiguous dimension.
//  * op() is addressing only ("Triton Optimization Reference", section 2):
//    a K-contiguous operand (A untransposed, B transposed) is staged with
//    rows along M/N and read into MFMA fragments with ds_read_b128; an
//    M/N-contiguous operand is staged as stored (rows along K) and read with
//    ds_read_b64_tr_b16, which transposes while reading.  Nothing is shuffled
//    in the loop.
//  * Tails: the buffer descriptor's size ends at the matrix's last element,
//    so rows past M/N or K read as zero in hardware.  Full K steps issue the
//    plain loads; only a final partial K step (K not a multiple of BK) also
//    points the K-contiguous units at or past K out of range, so they are
//    zero-filled (same page, section 1).  Columns past M/N inside a row are
//    read but only feed outputs that are never stored; only stores are
//    masked ("FLA Triton -> Gluon Porting Skill", pitfall 8: nothing in LDS
//    is left uninitialised).
//  * Pipeline (same page's prologue / steady state / epilogue skeleton):
//    STAGES-1 steps are in flight; at step kt a wave waits until its own
//    loads for kt have landed (vmcnt is an in-order counter, so "all but the
//    newest n loads" is exactly "step kt is done"), one barrier publishes
//    every wave's loads and retires step kt-1's buffer, then the loads for
//    step kt+STAGES-1 go into that buffer and the MFMAs consume step kt.
//  * v_mfma_f32_32x32x16 with fp32 accumulators in registers; each wave owns
//    (BM/WM) x (BN/WN) of the tile ("Finetuning Your Program": register
//    accumulator, many outputs per thread).
#pragma once

#include "common.hpp"

namespace tg {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14, expcnt in 6:4 left at its maximum, lgkmcnt in
// 11:8).  lgkmcnt(0) also retires this wave's LDS reads before a barrier
// lets other waves overwrite the buffer they read.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// Work-group barrier that orders memory operations only at compile time; the
// caller has already waited for whatever the other waves must see.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// One operand's DMA plan for one K step.  The LDS tile is ROWS x CH 16-byte
// units: KC (K-contiguous) tiles have MN_T rows of BK elements, the others
// BK rows of MN_T elements.  The tile is filled by INSTR wave instructions of
// 1 KiB, IPW per wave.
template <bool KC, int MN_T, int BK, int NW>
struct DmaOperand {
  static constexpr int CH = KC ? BK / 8 : MN_T / 8;
  static constexpr int BYTES = MN_T * BK * 2;
  static constexpr int INSTR = BYTES / 1024;
  static constexpr int IPW = INSTR / NW;
  static_assert(BYTES % 1024 == 0 && INSTR % NW == 0, "tile must split into whole 1 KiB wave loads");

  uint32_t voff[IPW];  // source byte offset from the tile's first element
  uint32_t kofs[IPW];  // K offset of the unit within the step (K-contiguous only)

  __device__ __forceinline__ void init(int wave, int lane, int64_t ld) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const uint32_t o = (uint32_t)(wave * IPW + i) * 1024u + 16u * lane;
      const uint32_t row = o / (CH * 16), phys = (o / 16) % CH;
      const uint32_t unit = phys ^ swz_unit<KC, CH>(row);
      voff[i] = (uint32_t)(((int64_t)row * ld + unit * 8) * 2);
      kofs[i] = KC ? unit * 8 : row;
    }
  }

  // base: element (mn0, k0) [KC] or (k0, mn0) [MN]; bytes: from base to the
  // end of the matrix's last element; k_left = K - k0.
  template <bool MASK_K>
  __device__ __forceinline__ void issue(const uint16_t* base, int64_t bytes, TG_LDS char* tile, int wave,
                                        int64_t k_left) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      uint32_t off = voff[i];
      if constexpr (MASK_K && KC) off = (int64_t)kofs[i] < k_left ? off : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TG_LDS void*)(tile + (wave * IPW + i) * 1024), 16, off, 0, 0,
                                               0);
    }
  }
};

template <typename In, typename Out, int BM, int BN, int BK, int WM, int WN, int STAGES, bool TA, bool TB>
__global__ void __launch_bounds__(WM * WN * 64) tile_gemm_kernel(GemmArgs args) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 16 == 0 && STAGES >= 2, "tile shape");
  constexpr bool A_KC = !TA, B_KC = TB;
  using OA = DmaOperand<A_KC, BM, BK, NW>;
  using OB = DmaOperand<B_KC, BN, BK, NW>;
  constexpr uint32_t A_BYTES = OA::BYTES, STAGE = OA::BYTES + OB::BYTES;
  constexpr int PER_STEP = OA::IPW + OB::IPW;  // vector-memory ops per wave per K step

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

  int32_t pm, pn;
  tile_coords<8>(blockIdx.x, args.tiles_m, args.tiles_n, pm, pn);
  const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
  const int64_t M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;

  OA oa;
  OB ob;
  oa.init(wave, lane, lda);
  ob.init(wave, lane, ldb);

  const int64_t nk = (K + BK - 1) / BK, nfull = K / BK;

  for (int64_t b = blockIdx.y; b < args.batch; b += gridDim.y) {
    const uint16_t* Ab = args.A + b * args.sA;
    const uint16_t* Bb = args.B + b * args.sB;

    auto issue = [&](int64_t kt) {
      const int64_t k0 = kt * BK;
      TG_LDS char* st = lds + (uint32_t)(kt % STAGES) * STAGE;
      const uint16_t* a0 = A_KC ? Ab + m0 * lda + k0 : Ab + k0 * lda + m0;
      const int64_t abytes = A_KC ? ((M - 1 - m0) * lda + (K - k0)) * 2 : ((K - 1 - k0) * lda + (M - m0)) * 2;
      const uint16_t* b0 = B_KC ? Bb + n0 * ldb + k0 : Bb + k0 * ldb + n0;
      const int64_t bbytes = B_KC ? ((N - 1 - n0) * ldb + (K - k0)) * 2 : ((K - 1 - k0) * ldb + (N - n0)) * 2;
      if (kt < nfull) {
        oa.template issue<false>(a0, abytes, st, wave, K - k0);
        ob.template issue<false>(b0, bbytes, st + A_BYTES, wave, K - k0);
      } else {
        oa.template issue<true>(a0, abytes, st, wave, K - k0);
        ob.template issue<true>(b0, bbytes, st + A_BYTES, wave, K - k0);
      }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(s);

    for (int64_t kt = 0; kt < nk; ++kt) {
      // loads issued after step kt that may stay in flight
      const int64_t ahead = min((int64_t)(STAGES - 2), nk - 1 - kt);
      if constexpr (STAGES >= 4) {
        if (ahead >= 2) wait_vmcnt<2 * PER_STEP>();
        else if (ahead == 1) wait_vmcnt<PER_STEP>();
        else wait_vmcnt<0>();
      } else if constexpr (STAGES == 3) {
        if (ahead >= 1) wait_vmcnt<PER_STEP>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      block_barrier();
      if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
      const TG_LDS char* sa = lds + (uint32_t)(kt % STAGES) * STAGE;
      mma_stage<In, FM, FN, BK, A_KC, B_KC, OA::CH, OB::CH>(sa, sa + A_BYTES, wm0, wn0, lane, acc);
    }

    void* Cb = (char*)args.C + b * args.sC * (int64_t)sizeof(Out);
    store_tile<Out, FM, FN>(Cb, args.ldc, M, N, m0 + wm0, n0 + wn0, lane, acc);
    if (b + gridDim.y < args.batch) {
      // the next matrix's prologue overwrites buffers other waves may still read
      wait_vmcnt<0>();
      block_barrier();
    }
  }
}

}  // namespace tg
