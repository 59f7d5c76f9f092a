// attention.hpp -- gfx950 fused attention forward pass:
//     O[b] = softmax(scale * Q[b] K[b]^T) V[b]      (row softmax, no mask)
//
// The two products are the attention-shaped pair the GEMM kernels run as
// separate batched launches (the pages' GEMM/BMM/attention reference,
// "Triton Optimization Reference (cuTile -> Triton)", opening section, names
// attention as the companion target of the same tiling rules).  Fused, the
// n_q x n_k score and probability matrices live only in registers: a
// work-group reads its Q rows once, streams K and V through LDS, and writes
// O once, so the pair's HBM traffic drops from ~4*n_q*n_k bytes per head to
// ~2*(n_q + 2*n_k)*d and the launch becomes bound by the matrix cores.
//
//  * Work: one work-group owns BM = 32*WAVES query rows of one head; each
//    wave owns 32 rows.  Work items are (head, row block) pairs decoded in
//    XCD-contiguous runs, so the row blocks of one head -- which all read
//    that head's K and V -- meet in one XCD's L2.
//  * Q: each lane keeps its query row's fragment for every 16-wide step of d
//    (8 elements, 16 bytes, per step) in registers for the whole item.
//  * K, V: BN keys at a time go HBM -> LDS by direct-to-LDS buffer loads into
//    a ring of S stages (the tile kernel's copy primitive and swizzles: K
//    rows are d-contiguous and read with ds_read_b128, V rows are read with
//    the transposing ds_read_b64_tr_b16).  Rows past n_k read as zero.
//  * Scores: v_mfma_f32_32x32x16 with K as the first operand and Q as the
//    second gives S^T: lane l holds query row l&31 and, per 32-key block,
//    keys 8g + 4(l>>5) + {0..3}, g = 0..3; lanes l and l^32 share a row.
//  * Online softmax: the running maximum m is kept in log2 units
//    (scale*log2(e)*score).  A block raises m only when some row's new
//    maximum exceeds m by more than TAU = 8, which is rare after the first
//    block; otherwise p = 2^(scale*log2e*s - m) <= 2^8 and nothing is
//    rescaled.  Any common m gives the same quotient, so this changes only
//    rounding.  Row sums accumulate per lane in fp32 and are combined with
//    the partner lane once at the end.
//  * P V: the probabilities are rounded to the input type (nearest even) and
//    used as the second MFMA operand straight from the score registers.  The
//    k order of that product is permuted to match the score layout (lane
//    half h supplies keys 16t + 4h + {0..3} and 16t + 8 + 4h + {0..3} of
//    16-key step t); the V fragment is read in the same order.
//  * Output: O is divided by the row sum and stored as fp32 or rounded to
//    the input type, rows past n_q dropped by the store descriptor.
#pragma once

#include "tile_gemm.hpp"

namespace tg {

struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  void* O;
  int64_t n_q, n_k;
  int64_t ldq, ldk, ldv, ldo;  // elements between rows
  int64_t sq, sk, sv, so;      // elements between heads
  int64_t batch;
  int32_t q_blocks;            // ceil(n_q / BM)
  float c;                     // scale * log2(e), > 0
};

using AttnFn = void (*)(AttnArgs);

// D: head dimension; WAVES: waves per work-group; RB: 32-row query blocks per
// wave (each K or V fragment read from LDS feeds RB MFMAs); BN: keys per
// stage; S: LDS stages.  RB = 1 runs two waves per SIMD (the softmax of one
// overlaps the MFMAs of the other); RB = 2 needs the whole register file
// (O alone is 128 registers per lane) and runs one.
template <typename In, typename Out, int D, int WAVES, int RB, int BN, int S>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 2 : 1)))
attn_fwd_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  static_assert(RB == 1 || RB == 2, "one or two row blocks per wave");
  static_assert(BN % 32 == 0 && S >= 2 && S <= 4, "stage shape");
  constexpr int WR = 32 * RB;            // query rows per wave
  constexpr int BM = WR * WAVES;         // query rows per work-group
  constexpr int ROWB = 2 * D;            // bytes of one K or V row
  constexpr int DCH = D / 8;             // 16-byte units per row
  constexpr int TI = BN * ROWB / 1024;   // 1 KiB wave copies per K (or V) tile
  static_assert(TI % WAVES == 0, "tile copies split evenly over the waves");
  constexpr int PW = TI / WAVES;         // per wave, per tile
  constexpr uint32_t TILE = BN * ROWB;
  constexpr uint32_t STAGE = 2 * TILE;   // K tile, then V tile
  constexpr int NKB = BN / 32;           // 32-key score blocks per stage
  constexpr int DS = D / 16;             // 16-wide d steps of Q K^T
  constexpr int DB = D / 32;             // 32-wide d blocks of O
  constexpr int KS = BN / 16;            // 16-key steps of P V
  constexpr float TAU = 8.f;             // log2 headroom before m is raised

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;
  const uint32_t lds0 = (uint32_t)(size_t)lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, lg = lane >> 5;
  const int trh = lane >> 4, trs = lane & 15;

  // this wave's share of a tile copy: instruction i covers tile bytes
  // (wave*PW + i)*1024 + 16*lane; the swizzle picks the source unit
  uint32_t koff[PW], voff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const uint32_t o = (uint32_t)(wave * PW + i) * 1024u + 16u * lane;
    const uint32_t row = o / ROWB, phys = (o / 16) % DCH;
    koff[i] = (uint32_t)(row * a.ldk * 2) + ((phys ^ swz_unit<true, DCH>(row)) << 4);
    voff[i] = (uint32_t)(row * a.ldv * 2) + ((phys ^ swz_unit<false, DCH>(row)) << 4);
  }

  const int64_t total = (int64_t)a.q_blocks * a.batch;
  const int64_t nkb = (a.n_k + BN - 1) / BN;

  for (int64_t w0 = blockIdx.x; w0 < total; w0 += gridDim.x) {
    int64_t b;
    int32_t qb, unused;
    work_coords<1>(w0, total, a.q_blocks, 1, b, qb, unused);
    const int64_t q0 = (int64_t)qb * BM;
    const int64_t rows_q = min((int64_t)BM, a.n_q - q0);
    const uint16_t* Kh = a.K + b * a.sk;
    const uint16_t* Vh = a.V + b * a.sv;

    // copies of key block j into stage s
    auto issue = [&](int64_t j, int s) {
      const int64_t k0 = j * BN;
      const int64_t valid = min((int64_t)BN, a.n_k - k0);
      const i32x4 rk = make_rsrc(Kh + k0 * a.ldk, ((valid - 1) * a.ldk + D) * 2);
      const i32x4 rv = make_rsrc(Vh + k0 * a.ldv, ((valid - 1) * a.ldv + D) * 2);
      const uint32_t st = lds0 + (uint32_t)s * STAGE + (uint32_t)(wave * PW) * 1024u;
#pragma unroll
      for (int i = 0; i < PW; ++i) dma16(rk, koff[i], st + (uint32_t)i * 1024u);
#pragma unroll
      for (int i = 0; i < PW; ++i) dma16(rv, voff[i], st + TILE + (uint32_t)i * 1024u);
    };

    // Q fragments of this lane's rows: row block rb, d = 16 ks + 8 lg .. +7
    u32x4 qf[RB][DS];
    {
      const __amdgpu_buffer_rsrc_t rq =
          store_rsrc(a.Q + b * a.sq + q0 * a.ldq, ((rows_q - 1) * a.ldq + D) * 2);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const uint32_t ro = (uint32_t)((wave * WR + rb * 32 + li) * a.ldq * 2);
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
          qf[rb][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rq, (int)(ro + (uint32_t)(16 * ks + 8 * lg) * 2), 0, 0));
      }
    }

#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nkb) issue(s, s);

    f32x16 o[RB][DB];
    float m[RB], l[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rb][i][r] = 0.f;
      m[rb] = -__builtin_inff();  // running maximum, log2 units
      l[rb] = 0.f;                // this lane's share of the row sum
    }

    for (int64_t j = 0; j < nkb; ++j) {
      // own copies of block j have landed (later blocks may still be in
      // flight); the barrier publishes everyone's and frees stage (j-1) % S
      wait_steps<2 * PW, true>(min((int64_t)(S - 2), nkb - 1 - j));
      block_barrier();
      if (j + S - 1 < nkb) issue(j + S - 1, (int)((j + S - 1) % S));
      const TG_LDS char* kt = lds + (uint32_t)(j % S) * STAGE;
      const TG_LDS char* vt = kt + TILE;

      // K fragments of the whole stage, all in flight before the first MFMA
      u32x4 kf[DS][NKB];
#pragma unroll
      for (int ks = 0; ks < DS; ++ks)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          kf[ks][kb] = lds_read16(kt, swz_off<true, DCH>(kb * 32 + li, ks * 16 + lg * 8));

      // scores S^T for BN keys x 32 query rows, per row block
      f32x16 sc[RB][NKB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[rb][kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DS; ++ks)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sc[rb][kb] = mfma32<In>(kf[ks][kb], qf[rb][ks], sc[rb][kb]);

      // V fragments, in flight while the softmax runs: lane half lg supplies
      // keys 16t + 4lg + {0..3} and 16t + 8 + 4lg + {0..3} of step t
      u32x4 vf[KS][DB];
#pragma unroll
      for (int t = 0; t < KS; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + 16 * (trh & 1) + 4 * (trs & 3);
          const int kr = t * 16 + 4 * lg + (trs >> 2);
          const u32x2 lo = lds_read_tr(vt, swz_off<false, DCH>(kr, col));
          const u32x2 hi = lds_read_tr(vt, swz_off<false, DCH>(kr + 8, col));
          vf[t][db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      __builtin_amdgcn_sched_barrier(0);

      // keys past n_k (last block only) take no weight; lane half lg holds
      // key kb*32 + 8(r>>2) + 4lg + (r&3) in register r
      const int valid = (int)min((int64_t)BN, a.n_k - j * BN);
      if (valid < BN) {
        const int thr = valid - 4 * lg;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + 8 * (r >> 2) + (r & 3) >= thr) sc[rb][kb][r] = -__builtin_inff();
      }

      u32x4 pf[RB][KS];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // row maximum over this block (both lane halves)
        float mx = sc[rb][0][0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[rb][kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxs = mx * a.c;
        if (__builtin_amdgcn_ballot_w64(mxs > m[rb] + TAU)) {
          const float mn = fmaxf(m[rb], mxs);
          const float alpha = __builtin_amdgcn_exp2f(m[rb] - mn);
          m[rb] = mn;
          l[rb] *= alpha;
#pragma unroll
          for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][i][r] *= alpha;
        }
        // probabilities (unnormalised) and their row sum (four partial sums)
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rb][kb][r], a.c, -m[rb]));
            ls[r & 3] += p[r];
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
            pf[rb][2 * kb + h] =
                u32x4{pack2<In>(p[8 * h], p[8 * h + 1]), pack2<In>(p[8 * h + 2], p[8 * h + 3]),
                      pack2<In>(p[8 * h + 4], p[8 * h + 5]), pack2<In>(p[8 * h + 6], p[8 * h + 7])};
        }
        l[rb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
      }
      __builtin_amdgcn_sched_barrier(0);

      // O += P V
#pragma unroll
      for (int t = 0; t < KS; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma32<In>(vf[t][db], pf[rb][t], o[rb][db]);
    }

    // normalise and store: register r of o[rb][db] is
    // O[row rb*32 + li][db*32 + 8(r>>2) + 4 lg + (r&3)]
    Out* Oh = (Out*)a.O + b * a.so + q0 * a.ldo;
    const __amdgpu_buffer_rsrc_t ro = store_rsrc(Oh, ((rows_q - 1) * a.ldo + D) * (int64_t)sizeof(Out));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float lt = l[rb] + __shfl_xor(l[rb], 32);
      const float inv = 1.f / lt;
      const uint32_t rowoff = (uint32_t)((wave * WR + rb * 32 + li) * a.ldo * (int64_t)sizeof(Out));
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t off = rowoff + (uint32_t)(db * 32 + 8 * g + 4 * lg) * (uint32_t)sizeof(Out);
          const float v0 = o[rb][db][4 * g] * inv, v1 = o[rb][db][4 * g + 1] * inv;
          const float v2 = o[rb][db][4 * g + 2] * inv, v3 = o[rb][db][4 * g + 3] * inv;
          if constexpr (sizeof(Out) == 4)
            buf_store16(ro, off, __builtin_bit_cast(u32x4, f32x4{v0, v1, v2, v3}));
          else
            buf_store8(ro, off, u32x2{pack2<Out>(v0, v1), pack2<Out>(v2, v3)});
        }
    }

    // every wave is done with the ring before the next item refills it
    if (w0 + gridDim.x < total) {
      wait_vmcnt<0>();
      block_barrier();
    }
  }
}

}  // namespace tg
