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
//  * Work items are (head, 256-row block) pairs decoded in XCD-contiguous
//    runs, so the row blocks of one head -- which all read that head's K and
//    V -- meet in one XCD's L2.
//  * Q: each lane keeps its query row's fragment for every 16-wide step of d
//    (8 elements, 16 bytes, per step) in registers for the whole item.
//  * K, V: 64 keys at a time go HBM -> LDS by direct-to-LDS buffer loads (the
//    tile kernel's copy primitive and swizzles: K rows are d-contiguous and
//    read with ds_read_b128, V rows are read with the transposing
//    ds_read_b64_tr_b16).  Rows past n_k read as zero.
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

// The kernel: eight waves in two groups of four; the dispatcher puts waves w
// and w + 4 on one SIMD, so each SIMD holds one wave of each group.  Wave w
// owns query rows [32 w, 32 w + 32) of a 256-row block.  A group alternates
// two phases, one work-group barrier after each:
//
//   MFMA phase i    : O += P(i-1) V(i-1), then S(i) = K(i) Q^T, with the V and
//                     K fragments read from LDS a few MFMAs ahead of use;
//   softmax phase i : the copies of key block i + 3, then the online softmax
//                     of S(i) into P(i) (registers only).
//
// Group 1 runs one phase behind group 0, so on every SIMD one wave issues
// back-to-back MFMAs while the other does the exponentials, and the matrix
// core waits only at the turn.  This is the pages' warp-specialised pipeline
// ("FLA Triton -> Gluon Porting Skill", section 5) with the two waves that
// share a SIMD, as the ping-pong GEMM kernel does for its copies.
//
//  * K blocks (64 keys) go through a ring of four LDS slots and V blocks
//    through a ring of five.  Every wave issues its share of block i + 3 in
//    its softmax phase i: K(i+3) into the slot of K(i-1), last read in group
//    1's MFMA phase i - 1, and V(i+3) into the slot of V(i-2), last read in
//    the same phase; both closed before the barrier that opened phase i.
//  * Before the barrier that ends global phase 2i + 1 every wave's share of
//    block i + 1 has landed: group 0 (end of its softmax phase i) may leave
//    blocks i + 2 and i + 3 in flight, group 1 (end of its MFMA phase i)
//    block i + 2.
//  * Registers: O (64), the Q fragments (32), S (32) and P (16) per lane; the
//    fragments in flight stay a few MFMAs deep, so nothing spills (a spill
//    reload would wait for every copy in flight).
template <typename In, typename Out, int D>
__global__ void __launch_bounds__(512) attn_pp_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  constexpr int NW = 8, BN = 64, RK = 4, RV = 5;  // waves, keys per block, ring slots
  constexpr int BM = 32 * NW;                     // query rows per work-group
  constexpr int ROWB = 2 * D;                     // bytes of one K or V row
  constexpr int DCH = D / 8;                      // 16-byte units per row
  constexpr int TI = BN * ROWB / 1024;            // 1 KiB wave copies per K (or V) block
  static_assert(TI % NW == 0, "block copies split evenly over the waves");
  constexpr int PW = TI / NW;                     // per wave, per block and operand
  constexpr int C = 2 * PW;                       // per wave, per block
  constexpr uint32_t TILE = BN * ROWB;
  constexpr int NKB = BN / 32;                    // 32-key score blocks
  constexpr int DS = D / 16;                      // 16-wide d steps of Q K^T
  constexpr int DB = D / 32;                      // 32-wide d blocks of O
  constexpr int KS = BN / 16;                     // 16-key steps of P V
  constexpr int NV = KS * DB, NK = DS * NKB;      // MFMAs of P V and of Q K^T
  constexpr int FP = 4;                           // fragments read ahead of their MFMA
  constexpr float TAU = 8.f;

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;
  const uint32_t lds0 = (uint32_t)(size_t)lds;  // K ring, then V ring

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int li = lane & 31, lg = lane >> 5;
  const int trh = lane >> 4, trs = lane & 15;

  uint32_t koff[PW], voff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const uint32_t o = (uint32_t)(wave * PW + i) * 1024u + 16u * lane;
    const uint32_t row = o / ROWB, phys = (o / 16) % DCH;
    koff[i] = (uint32_t)(row * a.ldk * 2) + ((phys ^ swz_unit<true, DCH>(row)) << 4);
    voff[i] = (uint32_t)(row * a.ldv * 2) + ((phys ^ swz_unit<false, DCH>(row)) << 4);
  }
  // LDS offsets of this lane's fragment reads: K step ks at rows li (+32 kb,
  // a constant), V block db at rows 4 lg + (trs >> 2) (+16 t and +8, constants:
  // the swizzles depend on the row only through bits the constants leave alone)
  uint32_t kof[DS], vof[DB];
#pragma unroll
  for (int ks = 0; ks < DS; ++ks) kof[ks] = swz_off<true, DCH>(li, ks * 16 + lg * 8);
#pragma unroll
  for (int db = 0; db < DB; ++db)
    vof[db] = swz_off<false, DCH>(4 * lg + (trs >> 2), db * 32 + 16 * (trh & 1) + 4 * (trs & 3));

  const int64_t total = (int64_t)a.q_blocks * a.batch;
  const int32_t nkb = (int32_t)((a.n_k + BN - 1) / BN);
  const bool ragged = a.n_k % BN != 0;

  for (int64_t w0 = blockIdx.x; w0 < total; w0 += gridDim.x) {
    int64_t b;
    int32_t qb, unused;
    work_coords<1>(w0, total, a.q_blocks, 1, b, qb, unused);
    const int64_t q0 = (int64_t)qb * BM;
    const int64_t rows_q = min((int64_t)BM, a.n_q - q0);
    // one resource per operand and head: rows at or past n_k lie past its
    // size and read as zero (the launcher keeps each head's span below 2 GiB,
    // so a block's byte offset rides in the 32-bit per-lane offset)
    const i32x4 rk = make_rsrc(a.K + b * a.sk, ((a.n_k - 1) * a.ldk + D) * 2);
    const i32x4 rv = make_rsrc(a.V + b * a.sv, ((a.n_k - 1) * a.ldv + D) * 2);
    const uint32_t kstep = (uint32_t)(BN * a.ldk * 2), vstep = (uint32_t)(BN * a.ldv * 2);

    auto issue = [&](int32_t j) __attribute__((always_inline)) {
      const uint32_t part = (uint32_t)(wave * PW) * 1024u;
      const uint32_t ks = lds0 + (uint32_t)(j % RK) * TILE + part;
      const uint32_t vs = lds0 + RK * TILE + (uint32_t)(j % RV) * TILE + part;
      const uint32_t kb = (uint32_t)j * kstep, vb = (uint32_t)j * vstep;
#pragma unroll
      for (int i = 0; i < PW; ++i) dma16(rk, koff[i] + kb, ks + (uint32_t)i * 1024u);
#pragma unroll
      for (int i = 0; i < PW; ++i) dma16(rv, voff[i] + vb, vs + (uint32_t)i * 1024u);
    };

    // Q fragments of this lane's row: d = 16 ks + 8 lg .. +7 (loaded before
    // the first copies, so the first counted wait covers them)
    u32x4 qf[DS];
    {
      const __amdgpu_buffer_rsrc_t rq =
          store_rsrc(a.Q + b * a.sq + q0 * a.ldq, ((rows_q - 1) * a.ldq + D) * 2);
      const uint32_t ro = (uint32_t)((wave * 32 + li) * a.ldq * 2);
#pragma unroll
      for (int ks = 0; ks < DS; ++ks)
        qf[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rq, (int)(ro + (uint32_t)(16 * ks + 8 * lg) * 2), 0, 0));
    }
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < nkb) issue(s);

    f32x16 o[DB], sc[NKB];
    u32x4 pf[KS];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
    float m = -__builtin_inff(), l = 0.f;

    // MFMA phase: MFMA q < NV is P V step (t, db) = (q / DB, q % DB) on
    // V(i-1); q >= NV is Q K^T step (ks, kb) on K(i).  Fragment q is read
    // FP MFMAs ahead.  WITH_PV / WITH_QK select the parts.
    auto mfma_phase = [&](int32_t i, auto with_pv, auto with_qk) __attribute__((always_inline)) {
      constexpr bool PV = decltype(with_pv)::value, QK = decltype(with_qk)::value;
      constexpr int Q0 = PV ? 0 : NV, Q1 = QK ? NV + NK : NV;
      // this phase's read bases, opaque to the compiler so that the constant
      // parts of the offsets stay in the instructions' offset fields
      const uint32_t vt = lds0 + RK * TILE + (uint32_t)((i + RV - 1) % RV) * TILE;
      const uint32_t kt = lds0 + (uint32_t)(i % RK) * TILE;
      uint32_t vb[DB], kb0[DS];
      if constexpr (PV) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          vb[db] = vt + vof[db];
          asm volatile("" : "+v"(vb[db]));
        }
      }
      if constexpr (QK) {
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
          kb0[ks] = kt + kof[ks];
          asm volatile("" : "+v"(kb0[ks]));
        }
      }
      u32x4 fr[NV + NK];
      auto load = [&](int q) __attribute__((always_inline)) {
        if (q < NV) {
          const int t = q / DB, db = q % DB;
          const TG_LDS char* v = (const TG_LDS char*)(size_t)vb[db];
          const u32x2 lo = lds_read_tr(v, (uint32_t)(t * 16 * ROWB));
          const u32x2 hi = lds_read_tr(v, (uint32_t)((t * 16 + 8) * ROWB));
          fr[q] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          const int ks = (q - NV) / NKB, kb = (q - NV) % NKB;
          fr[q] = lds_read16((const TG_LDS char*)(size_t)kb0[ks], (uint32_t)(kb * 32 * ROWB));
        }
      };
      if constexpr (QK) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
      }
#pragma unroll
      for (int q = Q0; q < Q0 + FP && q < Q1; ++q) load(q);
#pragma unroll
      for (int q = Q0; q < Q1; ++q) {
        if (q + FP < Q1) load(q + FP);
        if (q < NV) {
          const int t = q / DB, db = q % DB;
          o[db] = mfma32<In>(fr[q], pf[t], o[db]);
        } else {
          const int ks = (q - NV) / NKB, kb = (q - NV) % NKB;
          sc[kb] = mfma32<In>(fr[q], qf[ks], sc[kb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // softmax phase i: copies of block i + 3, then P(i) from S(i).  Keys
    // past n_k (a partial last block) take no weight; the branch is kept a
    // branch (the asm statement stops it being if-converted into selects
    // that every block would execute)
    auto softmax_phase = [&](int32_t i) __attribute__((always_inline)) {
      if (i + 3 < nkb) issue(i + 3);
      if (ragged && i == nkb - 1) {
        asm volatile("" ::: "memory");
        // opaque, so that the compare masks are not hoisted out of the loop
        // into scalar registers
        int thr = (int)(a.n_k - (int64_t)i * BN) - 4 * lg;
        asm volatile("" : "+v"(thr));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) >= thr) sc[kb][r] = -__builtin_inff();
      }
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      // A row's maximum exceeds m + TAU exactly when one of its two lanes'
      // halves does (scaling by c > 0 keeps the order), so the lanes decide
      // on their own halves and meet their partner only when m is raised.
      if (__builtin_amdgcn_ballot_w64(mx * a.c > m + TAU)) {
        asm volatile("" ::: "memory");  // a branch, not 64 multiplies per block
        const float mxs = fmaxf(mx, __shfl_xor(mx, 32)) * a.c;
        const float mn = fmaxf(m, mxs);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], a.c, -m));
          ls[r & 3] += p[r];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
          pf[2 * kb + h] = u32x4{pack2<In>(p[8 * h], p[8 * h + 1]), pack2<In>(p[8 * h + 2], p[8 * h + 3]),
                                 pack2<In>(p[8 * h + 4], p[8 * h + 5]), pack2<In>(p[8 * h + 6], p[8 * h + 7])};
      }
      l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };

    // counted waits: block i + 1 complete, `later` blocks' copies may stay
    // in flight; LDS reads drained
    auto wait_blocks = [&](int32_t later) __attribute__((always_inline)) {
      if (later >= 2) wait_vmcnt<2 * C, true>();
      else if (later == 1) wait_vmcnt<C, true>();
      else wait_vmcnt<0, true>();
    };

    // One key block for this wave: its MFMA phase and its softmax phase,
    // each closed by a barrier.  Group 0's MFMA phase i is global phase 2i,
    // group 1's is 2i + 1 (it opens with one extra barrier), so block i + 1
    // is complete before the barrier that ends global phase 2i + 1.  Each
    // group runs its own copy of the loop, with block 0 (no P V yet) peeled.
    auto step = [&](int32_t i, auto first, auto group) __attribute__((always_inline)) {
      mfma_phase(i, std::bool_constant<!decltype(first)::value>{}, std::true_type{});
      if constexpr (decltype(group)::value == 0)
        wait_vmcnt<63, true>();
      else
        wait_blocks(min(1, nkb - 2 - i));
      block_barrier();
      softmax_phase(i);
      if constexpr (decltype(group)::value == 0)
        wait_blocks(min(2, nkb - 2 - i));
      else
        wait_vmcnt<63, true>();
      block_barrier();
    };
    auto run = [&](auto group) __attribute__((always_inline)) {
      if constexpr (decltype(group)::value == 1) block_barrier();
      step(0, std::true_type{}, group);
      for (int32_t i = 1; i < nkb; ++i) step(i, std::false_type{}, group);
      mfma_phase(nkb, std::true_type{}, std::false_type{});
      if constexpr (decltype(group)::value == 0) block_barrier();
    };

    // block 0 (and the Q fragments) before the first phase
    wait_blocks(min(2, nkb - 1));
    block_barrier();
    if (grp == 0)
      run(std::integral_constant<int, 0>{});
    else
      run(std::integral_constant<int, 1>{});

    // normalise and store: register r of o[db] is
    // O[row li][db*32 + 8(r>>2) + 4 lg + (r&3)]
    Out* Oh = (Out*)a.O + b * a.so + q0 * a.ldo;
    const __amdgpu_buffer_rsrc_t ro = store_rsrc(Oh, ((rows_q - 1) * a.ldo + D) * (int64_t)sizeof(Out));
    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.f / lt;
    const uint32_t rowoff = (uint32_t)((wave * 32 + li) * a.ldo * (int64_t)sizeof(Out));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t off = rowoff + (uint32_t)(db * 32 + 8 * g + 4 * lg) * (uint32_t)sizeof(Out);
        const float v0 = o[db][4 * g] * inv, v1 = o[db][4 * g + 1] * inv;
        const float v2 = o[db][4 * g + 2] * inv, v3 = o[db][4 * g + 3] * inv;
        if constexpr (sizeof(Out) == 4)
          buf_store16(ro, off, __builtin_bit_cast(u32x4, f32x4{v0, v1, v2, v3}));
        else
          buf_store8(ro, off, u32x2{pack2<Out>(v0, v1), pack2<Out>(v2, v3)});
      }

    // every wave is done with the rings before the next item refills them
    if (w0 + gridDim.x < total) {
      wait_vmcnt<0>();
      block_barrier();
    }
  }
}

}  // namespace tg

