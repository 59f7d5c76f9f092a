// panel_gemm.hpp -- gfx950 GEMM/BMM for short K (K <= 128) with a K-contiguous
// A: products whose time goes into writing C.
//
// With K <= 128 a 128 x 128 tile of C needs at most 64 KiB of operands and
// 4.2 MFLOP but writes 64 KiB of fp32.  A work-group that loads, multiplies
// and stores one tile after another waits for each tile's operands with the
// previous tile's stores still ahead of them in the vector-memory counter
// (it retires in issue order), so every tile pays a load round trip behind a
// store drain.  Here a work-group walks a run of tiles along one row panel of
// C ("Triton Optimization Reference", section 7: persistent programs that
// loop over tiles):
//
//  * A's 128 x K panel is loaded once per run straight into the MFMA operand
//    registers -- lane l's 16-byte load is row (l mod 32) of a 32-row block
//    and the 8 consecutive k at 8 (l / 32) of a 16-deep slice -- and stays
//    there for the whole run (K <= 128: 64 registers).
//  * B's 128 x K tiles are copied HBM->LDS (buffer_load ... lds, the DMA
//    plan of the tile kernel) into two buffers.  The copy of tile t + 1 is
//    issued right after the barrier that opens tile t, before tile t's
//    stores, so the wait for it lets exactly those stores stay in flight.
//  * C goes out LDS-staged in 1 KiB row segments (store_tile_lds), staged in
//    the buffer tile t has just been read from.
//  * Runs: a row panel of tiles_n tiles, or a part of it when there would
//    otherwise be too few runs to fill the CUs (args.span tiles per run).
//    Run w0 goes to XCD w0 mod 8, each XCD taking a contiguous range of
//    (matrix, panel, part), so the panels of one matrix -- which all read
//    that matrix's B -- meet in one L2.
//
// The launcher sends only what this kernel serves: no epilogue, A stored
// M x K, 0 < K <= 128, 16-byte aligned operands with K, lda, ldb, ldc
// multiples of 8 and 128 rows of any operand within 2^31 bytes, and N a
// multiple of 16 bytes' worth of output elements.
#pragma once

#include "tile_gemm.hpp"
#include "tiles.hpp"

namespace tg {

template <typename In, typename Out, bool TB>
__global__ void __launch_bounds__(256, 2) panel_gemm_kernel(GemmArgs args) {
  constexpr int BM = kTiles[kPanelTile].bm, BN = kTiles[kPanelTile].bn, KMAX = kPanelKMax;
  constexpr int WM = 2, WN = 2, NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32, KS = KMAX / 16;
  constexpr bool B_KC = TB;
  using OB = DmaOperand<B_KC, BN, KMAX, NW>;
  constexpr uint32_t BUF = OB::BYTES;  // one B tile: 32 KiB
  constexpr uint32_t C_BYTES = (uint32_t)BM * BN * sizeof(Out);
  constexpr int PASSES = C_BYTES <= BUF ? 1 : WM;  // fp32 C goes out in two row bands
  static_assert(C_BYTES / PASSES <= BUF, "a staged band fits one B buffer");
  // store instructions per wave and tile (store_tile_lds: 16 bytes per thread each)
  constexpr int ST = BM * (BN * (int)sizeof(Out) / 16) / (NW * 64);
  static_assert(ST + OB::IPW < 64, "copies and stores in flight fit the vector-memory counter");

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;
  const uint32_t lds0 = (uint32_t)(size_t)lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
  const int li = lane & 31, lg = lane >> 5;
  const int trh = lane >> 4, trs = lane & 15;

  const int64_t M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb, ldc = args.ldc;
  const int32_t span = args.span;
  const int32_t parts = (args.tiles_n + span - 1) / span;
  const int64_t runs_per_matrix = (int64_t)args.tiles_m * parts;
  const int64_t total = runs_per_matrix * args.batch;

  OB ob;
  ob.init(wave, lane, ldb);
  // per-lane LDS offsets of the B fragment reads (slice ks, block j)
  uint32_t offb[KS][FN];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cb = wn0 + j * 32;
      if constexpr (B_KC)
        offb[ks][j] = swz_off<true, OB::CH>(cb + li, ks * 16 + lg * 8);
      else
        offb[ks][j] = swz_off<false, OB::CH>(ks * 16 + 8 * (trh >> 1) + (trs >> 2), cb + 16 * (trh & 1) + 4 * (trs & 3));
    }
  constexpr uint32_t B_TR4 = 4 * OB::CH * 16;  // the second transposing read is 4 rows further down

  for (int64_t w0 = blockIdx.x; w0 < total; w0 += gridDim.x) {
    const int64_t per = total >> 3, rem = total & 7, x = w0 & 7, local = w0 >> 3;
    const int64_t id = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
    const int64_t b = id / runs_per_matrix;
    const int32_t r = (int32_t)(id - b * runs_per_matrix);
    const int32_t pm = r / parts, part = r - pm * parts;
    const int32_t t0 = part * span, t1 = min(args.tiles_n, t0 + span);
    const int64_t m0 = (int64_t)pm * BM;

    // the previous run's staged C has been read by every wave before the
    // first copy of this run overwrites it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    block_barrier();

    // A panel -> operand registers; rows past M read zero (descriptor end),
    // slices past K get an out-of-range offset
    const uint16_t* Ab = args.A + b * args.sA + m0 * lda;
    const __amdgpu_buffer_rsrc_t ra = store_rsrc(Ab, ((M - 1 - m0) * lda + K) * 2);
    u32x4 fa[FM][KS];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = wm0 + 32 * i + li, k = 16 * ks + 8 * lg;
        const uint32_t off = k < K ? (uint32_t)(row * lda + k) * 2u : kOutOfRange;
        fa[i][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
      }

    const uint16_t* Bb = args.B + b * args.sB;
    auto copy_b = [&](int32_t pn, uint32_t buf) {
      const int64_t n0 = (int64_t)pn * BN;
      const uint16_t* base = Bb + (B_KC ? n0 * ldb : n0);
      const int64_t bytes = B_KC ? ((N - 1 - n0) * ldb + K) * 2 : ((K - 1) * ldb + (N - n0)) * 2;
      asm volatile("" ::: "memory");
      if (K < KMAX)
        ob.template issue<true>(base, bytes, lds0 + buf * BUF, wave, K);
      else
        ob.template issue<false>(base, bytes, lds0 + buf * BUF, wave, K);
      asm volatile("" ::: "memory");
    };
    copy_b(t0, 0);
    // the A registers and the first B tile (with whatever the previous run
    // left in flight)
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");

    for (int32_t t = t0; t < t1; ++t) {
      const uint32_t buf = (uint32_t)(t - t0) & 1u;
      if (t > t0) {
        // B(t) was issued before tile t-1's ST stores: only those may remain
        asm volatile("" ::: "memory");
        wait_vmcnt<ST>();
        asm volatile("" ::: "memory");
      }
      // B(t) is in LDS for every wave, and every wave has read tile t-1's
      // staged C out of the other buffer
      block_barrier();
      if (t + 1 < t1) copy_b(t + 1, buf ^ 1u);

      f32x16 acc[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
      const TG_LDS char* sb = lds + buf * BUF;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (16 * ks >= K) break;  // uniform: slices past K hold zeros
        u32x4 bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (B_KC) {
            bf[j] = lds_read16(sb, offb[ks][j]);
          } else {
            const u32x2 lo = lds_read_tr(sb, offb[ks][j]), hi = lds_read_tr(sb, offb[ks][j] + B_TR4);
            bf[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<In>(bf[j], fa[i][ks], acc[i][j]);
      }

      // every wave's fragment reads of this buffer are done before C is staged in it
      __builtin_amdgcn_s_waitcnt(0xC07F);
      block_barrier();
      const int64_t n0 = (int64_t)t * BN;
      char* Ct = (char*)args.C + (b * args.sC + m0 * ldc + n0) * (int64_t)sizeof(Out);
      const int64_t cbytes = ((M - 1 - m0) * ldc + (N - n0)) * (int64_t)sizeof(Out);
      asm volatile("" ::: "memory");
      if (args.stream_c)
        store_tile_lds<Out, BM, BN, WM, WN, FM, FN, PASSES, 2>(lds + buf * BUF, Ct, cbytes, ldc, N - n0, wave, lane,
                                                                acc);
      else
        store_tile_lds<Out, BM, BN, WM, WN, FM, FN, PASSES, 0>(lds + buf * BUF, Ct, cbytes, ldc, N - n0, wave, lane,
                                                                acc);
      asm volatile("" ::: "memory");
      // the staged C's LDS reads complete before the next barrier
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  }
}

}  // namespace tg
