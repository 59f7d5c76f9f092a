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

#include <type_traits>

namespace tg {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for raw (unstructured) loads: 48-bit base, no stride,
// `bytes` records (clamped below 2^31 so that kOutOfRange always misses), and
// the gfx9 default data-format word.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
  return i32x4{(int32_t)(uint32_t)a, (int32_t)((a >> 32) & 0xffffu), n, 0x00020000};
}

// One wave-wide 16-byte-per-lane HBM->LDS copy: lane t's 16 bytes at
// base + voff land at LDS byte address lds_addr + 16 t; offsets at or past
// the resource's size read as zero.  Issued as inline assembly so that the
// compiler neither waits on it before unrelated LDS reads nor reorders it
// across the explicit waits below: the kernel counts these loads itself.
// With `nt` the load carries the non-temporal hint: for operand bytes that
// no other tile of the launch reads, so that streaming them through the L2
// does not evict the lines other tiles still share.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr)
               : "m0");
}
__device__ __forceinline__ void dma16_nt(const i32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr)
               : "m0");
}
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t lds_addr, bool nt) {
  if (nt)
    dma16_nt(rsrc, voff, lds_addr);
  else
    dma16(rsrc, voff, lds_addr);
}

// s_waitcnt vmcnt(N), optionally with lgkmcnt(0) (gfx9 encoding: vmcnt[3:0]
// in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt in 6:4 left at its maximum,
// lgkmcnt in 11:8).  lgkmcnt(0) retires this wave's LDS reads, needed when
// the barrier that follows lets other waves overwrite the buffer just read.
template <int N, bool LGKM0 = true>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (LGKM0 ? 0 : (0xF << 8)));
}

// Run-time count (0 .. 2 steps' worth of loads); the counter field is an
// immediate, so dispatch over the few values a ring of <= 4 stages needs.
template <int PER_STEP, bool LGKM0>
__device__ __forceinline__ void wait_steps(int64_t steps) {
  if (steps >= 2) wait_vmcnt<2 * PER_STEP, LGKM0>();
  else if (steps == 1) wait_vmcnt<PER_STEP, LGKM0>();
  else wait_vmcnt<0, LGKM0>();
}

// As wait_steps, but EXTRA more operations (stores issued after the copies)
// may stay outstanding.
template <int PER_STEP, int EXTRA, int MAXSTEPS>
__device__ __forceinline__ void wait_steps_plus(int64_t steps) {
  // more than two steps are waited for as two (stricter, hence safe)
  static_assert(MAXSTEPS >= 0 && MAXSTEPS <= 2, "0 .. 2 steps");
  asm volatile("" ::: "memory");
  if constexpr (MAXSTEPS >= 2) {
    if (steps >= 2) {
      wait_vmcnt<2 * PER_STEP + EXTRA, true>();
      asm volatile("" ::: "memory");
      return;
    }
  }
  if constexpr (MAXSTEPS >= 1) {
    if (steps >= 1) {
      wait_vmcnt<PER_STEP + EXTRA, true>();
      asm volatile("" ::: "memory");
      return;
    }
  }
  wait_vmcnt<EXTRA, true>();
  asm volatile("" ::: "memory");
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

  // Instruction i of this wave's share (0 <= i < IPW).
  template <bool MASK_K>
  __device__ __forceinline__ void issue_one(int i, const i32x4& rs, uint32_t tile_lds, int wave, int64_t k_left,
                                            bool nt = false) const {
    uint32_t off = voff[i];
    if constexpr (MASK_K && KC) off = (int64_t)kofs[i] < k_left ? off : kOutOfRange;
    dma16(rs, off, tile_lds + (uint32_t)(wave * IPW + i) * 1024u, nt);
  }

  // base: element (mn0, k0) [KC] or (k0, mn0) [MN]; bytes: from base to the
  // end of the matrix's last element; k_left = K - k0.
  template <bool MASK_K>
  __device__ __forceinline__ void issue(const uint16_t* base, int64_t bytes, uint32_t tile_lds, int wave,
                                        int64_t k_left, bool nt = false) const {
    const i32x4 rs = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      uint32_t off = voff[i];
      if constexpr (MASK_K && KC) off = (int64_t)kofs[i] < k_left ? off : kOutOfRange;
      dma16(rs, off, tile_lds + (uint32_t)(wave * IPW + i) * 1024u, nt);
    }
  }
};

// ------------------------------------------------------------- epilogue ---
// Stores go through the compiler's builtins (not inline assembly) so that its
// hazard recognizer protects the store-data registers until they are read.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t rs, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t rs, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, rs, (int)off, 0, 0);
}
template <typename Out>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});  // nearest, ties to even
}
template <>
__device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}

// Vector store of a wave's FM x FN 32x32 blocks of C (acc holds C^T): every
// group of four registers is four consecutive columns of one row, written as
// one 16-byte (fp32) or 8-byte (16-bit) buffer store.  The descriptor's size
// ends at the last element of C, which drops rows past M; groups at or past
// column N get an out-of-range offset.  Needs N % 4 == 0 or a tile that ends
// inside N (the caller falls back to store_tile otherwise).
template <typename Out, int FM, int FN>
__device__ __forceinline__ void store_tile_vec(const void* Ctile, int64_t bytes, int64_t ldc, int64_t n_left,
                                               int lane, const f32x16 (&acc)[FM][FN]) {
  const __amdgpu_buffer_rsrc_t rs = store_rsrc(Ctile, bytes);
  const int li = lane & 31, lg = lane >> 5;
  constexpr uint32_t es = sizeof(Out);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const uint32_t rowoff = (uint32_t)((i * 32 + li) * ldc) * es;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = j * 32 + 8 * g + 4 * lg;
        const uint32_t off = col < n_left ? rowoff + (uint32_t)col * es : kOutOfRange;
        const f32x16& a = acc[i][j];
        if constexpr (sizeof(Out) == 4) {
          // (bit-cast the 4-vector as a whole: this compiler mislowers a bit
          // cast of a single vector element)
          buf_store16(rs, off, __builtin_bit_cast(u32x4, f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]}));
        } else {
          buf_store8(rs, off, u32x2{pack2<Out>(a[4 * g], a[4 * g + 1]), pack2<Out>(a[4 * g + 2], a[4 * g + 3])});
        }
      }
    }
  }
}

// The epilogue (alpha*acc + beta*C + bias, see epilogue_acc) with vector
// reads of C shaped like store_tile_vec's writes: per group of 4 registers,
// one 16-byte (fp32) or 8-byte (16-bit) load of 4 consecutive columns of one
// row.  Same descriptor and column mask as store_tile_vec (rows past M read
// zero, groups at or past n_left get an out-of-range offset); the bias is
// read element by element through a descriptor that ends at column N.
template <typename Out, int FM, int FN>
__device__ __forceinline__ void epilogue_acc_vec(const GemmArgs& args, const void* Ctile, int64_t bytes, int64_t ldc,
                                                 int64_t n_left, int64_t c0, int lane, f32x16 (&acc)[FM][FN]) {
  const int li = lane & 31, lg = lane >> 5;
  constexpr uint32_t es = sizeof(Out);
  const float alpha = args.alpha, beta = args.beta;
  float bias[FN][16];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[j][r] = 0.f;
  if (args.bias) {
    const __amdgpu_buffer_rsrc_t rb =
        store_rsrc((const char*)args.bias + c0 * (int64_t)es, n_left > 0 ? n_left * (int64_t)es : 0);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t off = (uint32_t)(j * 32 + 8 * (r >> 2) + 4 * lg + (r & 3)) * es;
        if constexpr (es == 4) {
          bias[j][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (int)off, 0, 0));
        } else {
          const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)off, 0, 0);
          bias[j][r] = (float)__builtin_bit_cast(Out, h);
        }
      }
  }
  const __amdgpu_buffer_rsrc_t rs = store_rsrc(Ctile, bytes);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const uint32_t rowoff = (uint32_t)((i * 32 + li) * ldc) * es;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = j * 32 + 8 * g + 4 * lg;
        float c[4] = {0.f, 0.f, 0.f, 0.f};
        if (beta != 0.f) {
          const uint32_t off = col < n_left ? rowoff + (uint32_t)col * es : kOutOfRange;
          // (whole-vector bit casts: this compiler mislowers a bit cast of
          // a single vector element)
          if constexpr (es == 4) {
            const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
#pragma unroll
            for (int q = 0; q < 4; ++q) c[q] = v[q];
          } else {
            typedef Out out4 __attribute__((ext_vector_type(4)));
            const out4 v = __builtin_bit_cast(out4, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0));
#pragma unroll
            for (int q = 0; q < 4; ++q) c[q] = (float)v[q];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 4 * g + q;
          acc[i][j][r] = __builtin_fmaf(beta, c[q], alpha * acc[i][j][r]) + bias[j][r];
        }
      }
    }
  }
}

// LDS-staged store of the work-group's BM x BN tile ("Triton Optimization
// Reference", section 5: the epilogue goes out in subtiles through shared
// memory).  The MFMA result layout gives each lane four consecutive columns
// of one row, so direct stores write 32 rows x 32 bytes per instruction --
// a scattered pattern the memory system handles poorly.  Here the waves
// first write their blocks (already converted to Out) into LDS, then every
// thread reads 16 consecutive bytes of a row and stores them, so one store
// instruction covers 1 KiB of whole row segments of C.  LDS rows are split
// into 16-byte units and unit u of row r sits at position u ^ (r & SM), which
// keeps the writes of 16 rows on distinct banks; the readers undo the XOR
// when they form the global column.  When the tile does not fit the LDS the
// kernel owns, it goes in PASSES row bands, one row of waves per band.
// Rows past M are dropped by the descriptor's size; 16-byte units at or past
// column N get an out-of-range offset (the caller guarantees N is a multiple
// of 16 / sizeof(Out)).
// LDS layout of a staged C band: rows of BN*sizeof(Out) bytes split into
// 16-byte units; unit u of row r sits at position u ^ (r & SM).
template <typename Out, int BN>
struct StagedC {
  static constexpr uint32_t es = sizeof(Out);
  static constexpr uint32_t ROWB = BN * es;  // bytes of one tile row
  static constexpr int UPR = ROWB / 16;      // 16-byte units per row
  static constexpr int SM = (UPR < 16 ? UPR : 16) - 1;
  static __device__ __forceinline__ uint32_t pos(int r, uint32_t byte) {
    return (uint32_t)r * ROWB + ((((byte >> 4) ^ (uint32_t)(r & SM))) << 4) + (byte & 15);
  }
};

// Waves whose rows fall in band `pass` (RP rows) write their blocks, already
// converted to Out, into the band's LDS image.
template <typename Out, int BM, int BN, int WM, int WN, int FM, int FN, int RP>
__device__ __forceinline__ void stage_c_write(TG_LDS char* lds, int pass, int wave, int lane,
                                              const f32x16 (&acc)[FM][FN]) {
  using L = StagedC<Out, BN>;
  const int li = lane & 31, lg = lane >> 5;
  const int wr = wave / WN, wn0 = (wave % WN) * (BN / WN);
  if (wr * (BM / WM) / RP != pass) return;
  const int rbase = wr * (BM / WM) - pass * RP;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = rbase + i * 32 + li;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn0 + j * 32 + 8 * g + 4 * lg;  // 4 consecutive columns
        const uint32_t at = L::pos(r, (uint32_t)col * L::es);
        const f32x16& a = acc[i][j];
        if constexpr (L::es == 4) {
          *(TG_LDS u32x4*)(lds + at) =
              __builtin_bit_cast(u32x4, f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]});
        } else {
          *(TG_LDS u32x2*)(lds + at) =
              u32x2{pack2<Out>(a[4 * g], a[4 * g + 1]), pack2<Out>(a[4 * g + 2], a[4 * g + 3])};
        }
      }
    }
  }
}

// Threads t = 0 .. NT-1 store the band: each reads 16 consecutive bytes of a
// row and writes them, so one store instruction covers 1 KiB of row segments.
template <typename Out, int BN, int RP, int NT, int AUX>
__device__ __forceinline__ void stage_c_store(const TG_LDS char* lds, __amdgpu_buffer_rsrc_t rs, int64_t ldc,
                                              int64_t n_left, int pass, int t) {
  using L = StagedC<Out, BN>;
  constexpr int UNITS = RP * L::UPR;
  static_assert(UNITS % NT == 0, "band splits evenly over the storing threads");
#pragma unroll
  for (int k = 0; k < UNITS / NT; ++k) {
    const int idx = k * NT + t;
    const int r = idx / L::UPR, p = idx % L::UPR;
    const u32x4 v = *(const TG_LDS u32x4*)(lds + (uint32_t)r * L::ROWB + (uint32_t)p * 16);
    const int u = p ^ (r & L::SM);
    const int col = u * (16 / L::es);
    const uint32_t off =
        col < n_left ? (uint32_t)((pass * RP + r) * ldc) * L::es + (uint32_t)col * L::es : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, AUX);
  }
}

// LDS-staged store of the work-group's BM x BN tile ("Triton Optimization
// Reference", section 5: the epilogue goes out in subtiles through shared
// memory).  The MFMA result layout gives each lane four consecutive columns
// of one row, so direct stores write 32 rows x 32 bytes per instruction --
// a scattered pattern the memory system handles poorly.  Here the waves
// first write their blocks (already converted to Out) into LDS, then every
// thread reads 16 consecutive bytes of a row and stores them, so one store
// instruction covers 1 KiB of whole row segments of C.  The XOR placement of
// 16-byte units keeps the writes of 16 rows on distinct banks; the readers
// undo it when they form the global column.  When the tile does not fit the
// LDS the kernel owns, it goes in PASSES row bands, one row of waves per
// band.  Rows past M are dropped by the descriptor's size; 16-byte units at
// or past column N get an out-of-range offset (the caller guarantees N is a
// multiple of 16 / sizeof(Out)).
template <typename Out, int BM, int BN, int WM, int WN, int FM, int FN, int PASSES, int AUX>
__device__ __forceinline__ void store_tile_lds(TG_LDS char* lds, void* Ctile, int64_t bytes, int64_t ldc,
                                               int64_t n_left, int wave, int lane, const f32x16 (&acc)[FM][FN]) {
  constexpr int NT = WM * WN * 64;
  constexpr int RP = BM / PASSES;  // rows per band
  static_assert(StagedC<Out, BN>::UPR >= 4 && RP % (BM / WM) == 0, "epilogue band shape");
  const __amdgpu_buffer_rsrc_t rs = store_rsrc(Ctile, bytes);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    stage_c_write<Out, BM, BN, WM, WN, FM, FN, RP>(lds, pass, wave, lane, acc);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    block_barrier();
    stage_c_store<Out, BN, RP, NT, AUX>(lds, rs, ldc, n_left, pass, wave * 64 + lane);
    if (pass + 1 < PASSES) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this band's LDS reads are done before the next band's writes
      block_barrier();
    }
  }
}

// Fragments of one 16-deep K slice for a wave's FM x FN blocks.
template <int FM, int FN>
struct Frags {
  u32x4 a[FM], b[FN];
};

// The kernel body.  KA is GemmArgs (one problem, or a batch of equal
// shapes) or, with GROUP, GroupArgs (a table of problems, each item looks its
// problem up; persistent modes and K rotation are off).  EPI compiles in the
// alpha/beta/bias epilogue; without it args.epi is ignored (the launcher
// sends epilogue calls to EPI entries), and the register allocator does not
// have to make room for the epilogue's C reads -- with them the HBM-bound
// 128 x 128 tile spilled, and its spill reloads, which wait for every copy
// in flight, slowed O = P V by 6-15%.
template <typename In, typename Out, int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int DW, bool TA,
          bool TB, bool GROUP, bool EPI, typename KA>
__device__ __forceinline__ void tile_gemm_body(const KA& kargs) {
  const GemmArgs& args = [&]() -> const GemmArgs& {
    if constexpr (GROUP) return kargs.g;
    else return kargs;
  }();
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KS = BK / 16;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 32 == 0 && STAGES >= 2 && STAGES <= 5, "tile shape");
  constexpr bool A_KC = !TA, B_KC = TB;
  // The last DW waves issue every HBM->LDS copy; with DW < NW the other waves
  // never stall on the texture path and keep the matrix cores fed.
  static_assert(DW >= 1 && DW <= NW, "copy waves");
  using OA = DmaOperand<A_KC, BM, BK, DW>;
  using OB = DmaOperand<B_KC, BN, BK, DW>;
  constexpr uint32_t A_BYTES = OA::BYTES, STAGE = OA::BYTES + OB::BYTES;
  constexpr int PER_STEP = OA::IPW + OB::IPW;  // copy instructions per copy wave per K step
  constexpr int READS = FM * (A_KC ? 1 : 2) + FN * (B_KC ? 1 : 2);  // LDS reads per 16-deep slice
  constexpr int MMAS = FM * FN;
  // Ring schedule.  A barrier at the start of every stage's last 16-deep
  // slice publishes stage kt + 1 (each wave first waits for its own copies),
  // and the copies for a later stage are interleaved with that slice's MFMAs.
  //  * With three or more buffers (EARLY) stage kt + STAGES - 1 goes into the
  //    buffer of stage kt - 1: every wave finished reading it before this
  //    barrier, so the barrier need not wait for this wave's own LDS reads.
  //  * With two buffers stage kt + 2 reuses stage kt's buffer, and the
  //    barrier must first retire this wave's reads of stage kt.
  constexpr bool EARLY = STAGES >= 3;
  constexpr int D = EARLY ? STAGES - 1 : STAGES;
  // LDS-staged epilogue: in one band if the tile fits the ring's LDS, else in
  // one band per row of waves; 0 = direct vector stores
  constexpr uint32_t C_BYTES = (uint32_t)BM * BN * sizeof(Out), RING_BYTES = STAGES * STAGE;
  constexpr int EPI_UPR = BN * (int)sizeof(Out) / 16;
  constexpr int EPI_P = C_BYTES <= RING_BYTES ? 1 : (C_BYTES / WM <= RING_BYTES ? WM : 0);
  constexpr int EPI_PASSES =
      (EPI_P > 0 && EPI_UPR >= 4 && ((BM / (EPI_P ? EPI_P : 1)) * EPI_UPR) % (NW * 64) == 0) ? EPI_P : 0;

  extern __shared__ __attribute__((aligned(1024))) char tg_smem[];
  TG_LDS char* lds = (TG_LDS char*)tg_smem;
  const uint32_t lds0 = (uint32_t)(size_t)lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
  const int li = lane & 31, lg = lane >> 5;
  const int trh = lane >> 4, trs = lane & 15;

  // the current item's problem (fixed for a plain launch)
  int64_t M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb, ldc = args.ldc;
  const uint16_t* Ap = args.A;
  const uint16_t* Bp = args.B;
  void* Cp = args.C;

  const int dwave = wave - (NW - DW);  // index among the copy waves (< 0: computes only)
  const bool copier = dwave >= 0;
  OA oa;
  OB ob;
  oa.init(copier ? dwave : 0, lane, lda);
  ob.init(copier ? dwave : 0, lane, ldb);

  // Per-lane LDS byte offsets of this wave's fragment reads for every slice
  // of a stage (the stage base is a compile-time immediate in steady state).
  uint32_t offa[KS][FM], offb[KS][FN];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm0 + i * 32;
      if constexpr (A_KC)
        offa[ks][i] = swz_off<true, OA::CH>(rb + li, ks * 16 + lg * 8);
      else
        offa[ks][i] = swz_off<false, OA::CH>(ks * 16 + 8 * (trh >> 1) + (trs >> 2), rb + 16 * (trh & 1) + 4 * (trs & 3));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cb = wn0 + j * 32;
      if constexpr (B_KC)
        offb[ks][j] = A_BYTES + swz_off<true, OB::CH>(cb + li, ks * 16 + lg * 8);
      else
        offb[ks][j] = A_BYTES + swz_off<false, OB::CH>(ks * 16 + 8 * (trh >> 1) + (trs >> 2),
                                                       cb + 16 * (trh & 1) + 4 * (trs & 3));
    }
  }
  // the second transposing read of a fragment is 4 rows further down
  constexpr uint32_t A_TR4 = 4 * OA::CH * 16, B_TR4 = 4 * OB::CH * 16;

  int64_t nk = (K + BK - 1) / BK, nfull = K / BK;
  // bytes the loads of one operand advance per K step
  int64_t a_step = A_KC ? (int64_t)BK * 2 : (int64_t)BK * lda * 2;
  int64_t b_step = B_KC ? (int64_t)BK * 2 : (int64_t)BK * ldb * 2;

  // Walk order over the K steps.  Normally 0, 1, ...; with rotate_k the
  // full steps are walked from a per-work-group starting step (the partial
  // step, if any, stays last).  Work-groups otherwise run in lock-step and,
  // when each streams an operand panel of its own, all of them hit the same
  // offsets -- and HBM channels -- at the same time.  Tiles that share
  // panels (grouped launch order) keep the plain order so that neighbours
  // still meet in L2.
  int64_t total;
  if constexpr (GROUP) total = kargs.total;
  else total = (int64_t)args.tiles_m * args.tiles_n * args.batch;
  // Persistent mode (args.persist): a work-group walks several items and,
  // once an item's K loop is done, issues the next item's prologue copies
  // before this item's stores, so the next K loop starts while the stores
  // drain.  Loads and stores retire through one in-order counter, so the
  // first wait of a prefetched item lets exactly ST later operations -- the
  // stores, a fixed count per wave -- stay outstanding.
  constexpr int ST = FM * FN * 4;  // store instructions of store_tile_vec
  constexpr bool PERSIST_OK = (D - 1) * PER_STEP + ST < 64;  // fits the counter
  const bool persist = !GROUP && PERSIST_OK && args.persist == 1 && !(EPI && args.epi);
  // the item being computed: matrix, tile origin, walk rotation, and the
  // source pointers / remaining bytes / K - k0 of the next step to load
  int64_t b = 0, m0 = 0, n0 = 0, rot = 0;
  const char* a_base = nullptr;
  const char* b_base = nullptr;
  int64_t a_left0 = 0, b_left0 = 0;
  const char* a_ptr = nullptr;
  const char* b_ptr = nullptr;
  int64_t a_left = 0, b_left = 0, k_left = 0;
  int64_t ld_step = 0;  // walk position of the next step to load
  auto seek = [&]() {
    int64_t p = ld_step;
    if (ld_step < nfull) {
      p += rot;
      p = p >= nfull ? p - nfull : p;
    }
    a_ptr = a_base + p * a_step;
    a_left = a_left0 - p * a_step;
    b_ptr = b_base + p * b_step;
    b_left = b_left0 - p * b_step;
    k_left = K - p * BK;
  };
  auto setup = [&](int64_t w) {
    int32_t pm, pn;
    if constexpr (GROUP) {
      // XCD x (work-groups w = x mod 8) takes a contiguous run of items, so
      // the tiles of one problem, which share its operands, meet in one L2
      const int64_t per = total >> 3, rem = total & 7, x = w & 7, local = w >> 3;
      const int64_t id = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
      // the item's problem: the last one whose first item is <= id
      int32_t q = 0;
      for (int32_t i = 1; i < kargs.count; ++i)
        if (kargs.p[i].first <= id) q = i;
      const GroupProblem& pr = kargs.p[q];
      M = pr.M;
      N = pr.N;
      K = pr.K;
      lda = pr.lda;
      ldb = pr.ldb;
      ldc = pr.ldc;
      Ap = pr.A;
      Bp = pr.B;
      Cp = pr.C;
      nk = (K + BK - 1) / BK;
      nfull = K / BK;
      a_step = A_KC ? (int64_t)BK * 2 : (int64_t)BK * lda * 2;
      b_step = B_KC ? (int64_t)BK * 2 : (int64_t)BK * ldb * 2;
      oa.init(copier ? dwave : 0, lane, lda);
      ob.init(copier ? dwave : 0, lane, ldb);
      // column-major tiles: the row tiles of one B panel are neighbours
      const int32_t t = (int32_t)(id - pr.first), tm = (int32_t)((M + BM - 1) / BM);
      pn = t / tm;
      pm = t - pn * tm;
      b = 0;
    } else {
      work_coords<8>(w, total, args.tiles_m, args.tiles_n, b, pm, pn);
    }
    m0 = (int64_t)pm * BM;
    n0 = (int64_t)pn * BN;
    rot = (!GROUP && args.rotate_k && nfull > 1) ? w % nfull : 0;
    a_base = (const char*)(Ap + b * args.sA + (A_KC ? m0 * lda : m0));
    b_base = (const char*)(Bp + b * args.sB + (B_KC ? n0 * ldb : n0));
    a_left0 = A_KC ? ((M - 1 - m0) * lda + K) * 2 : ((K - 1) * lda + (M - m0)) * 2;
    b_left0 = B_KC ? ((N - 1 - n0) * ldb + K) * 2 : ((K - 1) * ldb + (N - n0)) * 2;
    ld_step = 0;
    seek();
  };
  // operands no other tile of the launch reads are loaded non-temporally
  const bool nt_a = !GROUP && (args.nt_ab & 1), nt_b = !GROUP && (args.nt_ab & 2);
  bool prefetched = false;  // this item's prologue copies were issued by the previous item
  bool behind_stores = false;  // ... and this wave's stores of that item were issued after them

  for (int64_t w0 = blockIdx.x; w0 < total; w0 += gridDim.x) {
    if (!prefetched) setup(w0);

    auto issue = [&](uint32_t buf, auto full) {
      const uint32_t st = lds0 + buf * STAGE;
      if (!copier) {
      } else if (decltype(full)::value || k_left >= BK) {
        oa.template issue<false>((const uint16_t*)a_ptr, a_left, st, dwave, k_left, nt_a);
        ob.template issue<false>((const uint16_t*)b_ptr, b_left, st + A_BYTES, dwave, k_left, nt_b);
      } else {
        oa.template issue<true>((const uint16_t*)a_ptr, a_left, st, dwave, k_left, nt_a);
        ob.template issue<true>((const uint16_t*)b_ptr, b_left, st + A_BYTES, dwave, k_left, nt_b);
      }
      ++ld_step;
      seek();
    };

    // LDS -> registers: read r (0 <= r < READS) of slice ks of the stage at
    // byte `base`; A fragments first, then B, two transposing reads per
    // M/N-contiguous fragment.
    auto read_one = [&](uint32_t base, int ks, int r, Frags<FM, FN>& f) {
      const TG_LDS char* sb = lds + base;
      constexpr int RA = FM * (A_KC ? 1 : 2);
      if (r < RA) {
        if constexpr (A_KC) {
          f.a[r] = lds_read16(sb, offa[ks][r]);
        } else {
          const int i = r >> 1;
          const u32x2 v = lds_read_tr(sb, offa[ks][i] + ((r & 1) ? A_TR4 : 0u));
          f.a[i][(r & 1) * 2] = v[0];
          f.a[i][(r & 1) * 2 + 1] = v[1];
        }
      } else {
        const int q = r - RA;
        if constexpr (B_KC) {
          f.b[q] = lds_read16(sb, offb[ks][q]);
        } else {
          const int j = q >> 1;
          const u32x2 v = lds_read_tr(sb, offb[ks][j] + ((q & 1) ? B_TR4 : 0u));
          f.b[j][(q & 1) * 2] = v[0];
          f.b[j][(q & 1) * 2 + 1] = v[1];
        }
      }
    };
    auto read = [&](uint32_t base, int ks, Frags<FM, FN>& f) {
#pragma unroll
      for (int r = 0; r < READS; ++r) read_one(base, ks, r, f);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // One 16-deep slice in a fixed instruction order: MFMA m, then the m-th
    // LDS read for the next slice, then (evenly spaced) one HBM->LDS copy of
    // this wave's instructions [d0, d0 + cnt) for a later stage, so that
    // neither the LDS nor the vector-memory path sees a burst.
    // sched_barrier(0) pins the order.
    auto dma_one = [&](int d, const i32x4& ra, const i32x4& rb, uint32_t dst) {
      if (!copier) return;
      if (d < OA::IPW)
        oa.template issue_one<false>(d, ra, dst, dwave, BK, nt_a);
      else
        ob.template issue_one<false>(d - OA::IPW, rb, dst + A_BYTES, dwave, BK, nt_b);
    };
    auto slice = [&](const Frags<FM, FN>& cur, Frags<FM, FN>* nxt, uint32_t nbase, int nks, const i32x4* rsa,
                     const i32x4* rsb, uint32_t dma_st, int d0, int cnt) {
      const int every = cnt > 0 ? (MMAS / cnt > 0 ? MMAS / cnt : 1) : MMAS;
      int d = 0;
#pragma unroll
      for (int m = 0; m < MMAS; ++m) {
        const int i = m / FN, j = (i & 1) ? FN - 1 - m % FN : m % FN;  // snake order
        acc[i][j] = mfma32<In>(cur.b[j], cur.a[i], acc[i][j]);
        if (nxt && m < READS) read_one(nbase, nks, m, *nxt);
        if (rsa && m % every == every - 1 && d < cnt) {
          dma_one(d0 + d, *rsa, *rsb, dma_st);
          ++d;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (nxt) {
#pragma unroll
        for (int r = MMAS; r < READS; ++r) read_one(nbase, nks, r, *nxt);
      }
      if (rsa) {
#pragma unroll
        for (; d < cnt; ++d) dma_one(d0 + d, *rsa, *rsb, dma_st);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto mma = [&](const Frags<FM, FN>& f) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          const int j = (i & 1) ? FN - 1 - jj : jj;  // snake order
          acc[i][j] = mfma32<In>(f.b[j], f.a[i], acc[i][j]);
        }
    };

    if (nk > 0) {
      Frags<FM, FN> f[2];
      if (!prefetched) {
#pragma unroll
        for (int s = 0; s < D; ++s)
          if (s < nk) issue((uint32_t)s, std::false_type{});
      }
      if (behind_stores) {
        if constexpr (PERSIST_OK) wait_steps_plus<PER_STEP, ST, (D - 1 < 2 ? D - 1 : 2)>(min((int64_t)D, nk) - 1);
      } else if (copier) {
        wait_steps<PER_STEP, true>(min((int64_t)D, nk) - 1);
      } else {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // no copies of its own: only its LDS reads
      }
      block_barrier();
      read(0, 0, f[0]);

      // One stage held in buffer `buf`: KS slices; the last slice crosses to
      // the next stage after the wait + barrier that publishes stage kt + 1.
      auto stage_const = [&](auto bufc) {
        constexpr uint32_t buf = decltype(bufc)::value;
        constexpr uint32_t dst = ((buf + D) % STAGES) * STAGE;
        const i32x4 rsa = make_rsrc(a_ptr, a_left), rsb = make_rsrc(b_ptr, b_left);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frags<FM, FN>& cur = f[ks & 1];
          Frags<FM, FN>& nxt = f[(ks & 1) ^ 1];
          if (ks + 1 < KS) {
            slice(cur, &nxt, buf * STAGE, ks + 1, nullptr, nullptr, 0, 0, 0);
          } else {
            // copies for stages kt+2 .. kt+D-1 may stay in flight
            if (DW == NW || copier) wait_vmcnt<(D - 2) * PER_STEP, !EARLY>();
            else if constexpr (!EARLY) __builtin_amdgcn_s_waitcnt(0xC07F);
            block_barrier();
            slice(cur, &nxt, ((buf + 1) % STAGES) * STAGE, 0, &rsa, &rsb, lds0 + dst, 0, PER_STEP);
          }
        }
        ++ld_step;
        seek();
      };
      auto stage_dyn = [&](int64_t kt) {
        const uint32_t buf = (uint32_t)(kt % STAGES);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frags<FM, FN>& cur = f[ks & 1];
          Frags<FM, FN>& nxt = f[(ks & 1) ^ 1];
          if (ks + 1 < KS) {
            read(buf * STAGE, ks + 1, nxt);
          } else if (kt + 1 < nk) {
            if (behind_stores && kt + 1 < D) {
              // stage kt+1 was issued before the previous item's ST stores,
              // which may still be in flight behind it
              if constexpr (PERSIST_OK)
                wait_steps_plus<PER_STEP, ST, (D - 2 < 2 ? D - 2 : 2)>(min((int64_t)(D - 2), nk - 2 - kt));
            } else if (DW == NW || copier) {
              wait_steps<PER_STEP, !EARLY>(min((int64_t)(D - 2), nk - 2 - kt));
            } else if constexpr (!EARLY) {
              __builtin_amdgcn_s_waitcnt(0xC07F);
            }
            block_barrier();
            if (kt + D < nk) issue((uint32_t)((kt + D) % STAGES), std::false_type{});
            read((uint32_t)((kt + 1) % STAGES) * STAGE, 0, nxt);
          }
          mma(cur);
        }
      };
      // steady state: groups of STAGES stages (compile-time buffers) whose
      // loads are all full K steps
      const int64_t nsteady = max((int64_t)0, min(nk, nfull) - D);
      int64_t kt = 0;
      if (behind_stores) {
        // the first stages' waits must allow for the previous item's stores;
        // one ring's worth of stages keeps the steady loop's buffers aligned
        const int64_t head = min((int64_t)STAGES, nk);
        for (; kt < head; ++kt) stage_dyn(kt);
      }
      for (; kt + STAGES <= nsteady; kt += STAGES) {
        stage_const(std::integral_constant<uint32_t, 0>{});
        stage_const(std::integral_constant<uint32_t, 1>{});
        if constexpr (STAGES > 2) stage_const(std::integral_constant<uint32_t, 2>{});
        if constexpr (STAGES > 3) stage_const(std::integral_constant<uint32_t, 3>{});
        if constexpr (STAGES > 4) stage_const(std::integral_constant<uint32_t, 4>{});
      }
      for (; kt < nk; ++kt) stage_dyn(kt);
    }

    if (!GROUP && EPI && args.epi) {
      const char* Cb = (const char*)Cp + b * args.sC * (int64_t)sizeof(Out);
      const int64_t r0 = m0 + wm0, c0 = n0 + wn0;
      if (N % 4 == 0 || n0 + BN <= N) {  // 4-column groups never straddle column N
        if (r0 < M && c0 < N)
          epilogue_acc_vec<Out, FM, FN>(args, Cb + (r0 * ldc + c0) * (int64_t)sizeof(Out),
                                        ((M - 1 - r0) * ldc + (N - c0)) * (int64_t)sizeof(Out), ldc, N - c0, c0,
                                        lane, acc);
      } else {
        epilogue_acc<Out, FM, FN>(args, Cb, ldc, M, N, r0, c0, lane, acc);
      }
    }
    // this item's origin (in persistent mode the state moves on below)
    const int64_t cb = b, cm0 = m0, cn0 = n0;
    prefetched = false;
    behind_stores = false;
    if (persist && w0 + gridDim.x < total) {
      // every wave's LDS reads of this item are done before the ring is
      // refilled with the next item's first stages
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      block_barrier();
      setup(w0 + gridDim.x);
      if (nk > 0) {
#pragma unroll
        for (int s = 0; s < D; ++s)
          if (s < nk) issue((uint32_t)s, std::false_type{});
      }
      prefetched = true;
      behind_stores = true;
      asm volatile("" ::: "memory");
    }
    {
      const int64_t r0 = cm0 + wm0, c0 = cn0 + wn0;
      char* Cb = (char*)Cp + cb * args.sC * (int64_t)sizeof(Out);
      if (persist) {
        // always ST store instructions (waves outside C store nothing: an
        // empty descriptor drops every access)
        const bool in = r0 < M && c0 < N;
        store_tile_vec<Out, FM, FN>(in ? Cb + (r0 * ldc + c0) * (int64_t)sizeof(Out) : Cb,
                                    in ? ((M - 1 - r0) * ldc + (N - c0)) * (int64_t)sizeof(Out) : 0, ldc,
                                    in ? N - c0 : 0, lane, acc);
        goto stored;
      }
      if constexpr (EPI_PASSES > 0) {
        if (N % (16 / (int)sizeof(Out)) == 0) {  // uniform over the work-group
          // every wave's reads of the last stage are done before LDS is reused
          __builtin_amdgcn_s_waitcnt(0xC07F);
          block_barrier();
          // non-temporal stores (args.stream_c) for outputs far larger than
          // the L2s, so that they do not evict the operands' panels
          if (args.stream_c)
            store_tile_lds<Out, BM, BN, WM, WN, FM, FN, EPI_PASSES, 2>(
                lds, Cb + (cm0 * ldc + cn0) * (int64_t)sizeof(Out),
                ((M - 1 - cm0) * ldc + (N - cn0)) * (int64_t)sizeof(Out), ldc, N - cn0, wave, lane, acc);
          else
            store_tile_lds<Out, BM, BN, WM, WN, FM, FN, EPI_PASSES, 0>(
                lds, Cb + (cm0 * ldc + cn0) * (int64_t)sizeof(Out),
                ((M - 1 - cm0) * ldc + (N - cn0)) * (int64_t)sizeof(Out), ldc, N - cn0, wave, lane, acc);
          goto stored;
        }
      }
      if (N % 4 == 0 || cn0 + BN <= N) {
        if (r0 < M && c0 < N)
          store_tile_vec<Out, FM, FN>(Cb + (r0 * ldc + c0) * (int64_t)sizeof(Out),
                                      ((M - 1 - r0) * ldc + (N - c0)) * (int64_t)sizeof(Out), ldc, N - c0,
                                      lane, acc);
      } else {
        store_tile<Out, FM, FN>(Cb, ldc, M, N, r0, c0, lane, acc);
      }
    stored:;
    }
    if (!persist && w0 + gridDim.x < total) {
      // the next tile's prologue overwrites buffers other waves may still read
      wait_vmcnt<0>();
      block_barrier();
    }
  }
}

template <typename In, typename Out, int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int DW, bool TA, bool TB,
          bool EPI>
__global__ void __launch_bounds__(WM * WN * 64, OCC * WM * WN / 4) tile_gemm_kernel(GemmArgs args) {
  tile_gemm_body<In, Out, BM, BN, BK, WM, WN, STAGES, OCC, DW, TA, TB, false, EPI>(args);
}

template <typename In, typename Out, int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int DW, bool TA, bool TB>
__global__ void __launch_bounds__(WM * WN * 64, OCC * WM * WN / 4) group_gemm_kernel(GroupArgs args) {
  tile_gemm_body<In, Out, BM, BN, BK, WM, WN, STAGES, OCC, DW, TA, TB, true, false>(args);
}

}  // namespace tg
