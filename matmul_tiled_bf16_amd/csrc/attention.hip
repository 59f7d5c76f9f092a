// attention.hip -- kernel instances and the C ABI of the fused attention
// forward pass declared in include/tgemm.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "../../include/tgemm.h"
#include "attention.hpp"

namespace {

using tg::AttnArgs;
using tg::AttnFn;

// One launch shape per head dimension: the ping-pong kernel's 8 waves of 32
// query rows (256 per work-group), 64-key blocks, rings of 4 K and 5 V blocks
// (144 KiB of LDS at d = 128: one work-group per CU).
constexpr int kWaves = 8, kBN = 64, kRingK = 4, kRingV = 5;

template <typename In, typename Out, int D>
constexpr AttnFn attn_kernel() {
  return tg::attn_pp_kernel<In, Out, D>;
}

// [in bf16/fp16][out fp32/same][d 64/128]
const AttnFn kAttn[2][2][2] = {
    {{attn_kernel<__bf16, float, 64>(), attn_kernel<__bf16, float, 128>()},
     {attn_kernel<__bf16, __bf16, 64>(), attn_kernel<__bf16, __bf16, 128>()}},
    {{attn_kernel<_Float16, float, 64>(), attn_kernel<_Float16, float, 128>()},
     {attn_kernel<_Float16, _Float16, 64>(), attn_kernel<_Float16, _Float16, 128>()}}};

constexpr uint32_t lds_bytes(int d) { return (uint32_t)(kRingK + kRingV) * kBN * 2u * (uint32_t)d; }

}  // namespace

extern "C" {

tg_status attention_fwd(tg_dtype in_type, tg_dtype out_type, int64_t batch, int64_t n_q, int64_t n_k,
                        int64_t head_dim, float scale, const void* Q, int64_t ldq, int64_t stride_q, const void* K,
                        int64_t ldk, int64_t stride_k, const void* V, int64_t ldv, int64_t stride_v, void* O,
                        int64_t ldo, int64_t stride_o, hipStream_t stream) {
  if (batch < 0 || n_q < 0 || n_k < 0 || head_dim < 1) return TG_ERR_INVALID;
  if (!(std::isfinite(scale) && scale > 0.f)) return TG_ERR_INVALID;
  if (ldq < head_dim || ldk < head_dim || ldv < head_dim || ldo < head_dim) return TG_ERR_INVALID;
  if (stride_q < 0 || stride_k < 0 || stride_v < 0 || stride_o < 0) return TG_ERR_INVALID;
  if (in_type != TG_BF16 && in_type != TG_FP16) return TG_ERR_UNSUPPORTED;
  if (out_type != TG_FP32 && out_type != in_type) return TG_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return TG_ERR_UNSUPPORTED;
  if (batch == 0 || n_q == 0) return TG_OK;
  if (n_k == 0) return TG_ERR_INVALID;  // a softmax over no keys is undefined
  if (!Q || !K || !V || !O) return TG_ERR_INVALID;
  // every head's rows must stay far inside int64 element offsets; the
  // kernels' 31-bit buffer offsets span at most 128 rows of any operand
  const int64_t big = (int64_t)1 << 60;
  if (n_q > big / ldq || n_k > big / ldk || n_k > big / ldv || n_q > big / ldo) return TG_ERR_INVALID;
  if (batch > 1 && (stride_q > big / batch || stride_k > big / batch || stride_v > big / batch ||
                    stride_o > big / batch))
    return TG_ERR_INVALID;
  if (batch > 1 && stride_o < (n_q - 1) * ldo + head_dim) return TG_ERR_INVALID;  // heads' outputs overlap
  const int64_t lim = (int64_t)1 << 20;
  if (ldq >= lim || ldk >= lim || ldv >= lim || ldo >= lim) return TG_ERR_UNSUPPORTED;
  // the kernel addresses a head's K and V through one buffer resource each,
  // with 32-bit byte offsets
  const int64_t span = (int64_t)1 << 30;
  if ((n_k - 1) * ldk + head_dim >= span || (n_k - 1) * ldv + head_dim >= span) return TG_ERR_UNSUPPORTED;
  // 16-byte loads and stores along d
  const bool aligned = (uintptr_t)Q % 16 == 0 && (uintptr_t)K % 16 == 0 && (uintptr_t)V % 16 == 0 &&
                       (uintptr_t)O % 16 == 0 && ldq % 8 == 0 && ldk % 8 == 0 && ldv % 8 == 0 && ldo % 8 == 0 &&
                       (batch == 1 || (stride_q % 8 == 0 && stride_k % 8 == 0 && stride_v % 8 == 0 &&
                                       stride_o % 8 == 0));
  if (!aligned) return TG_ERR_UNSUPPORTED;

  constexpr int BM = 32 * kWaves;
  const int64_t q_blocks = (n_q + BM - 1) / BM;
  if (q_blocks >= ((int64_t)1 << 31)) return TG_ERR_INVALID;
  const int64_t total = q_blocks * batch;

  AttnArgs a;
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.O = O;
  a.n_q = n_q;
  a.n_k = n_k;
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.ldo = ldo;
  a.sq = stride_q;
  a.sk = stride_k;
  a.sv = stride_v;
  a.so = stride_o;
  a.batch = batch;
  a.q_blocks = (int32_t)q_blocks;
  a.c = (float)((double)scale * 1.4426950408889634074);  // log2(e)

  const int io = in_type == TG_BF16 ? 0 : 1, oo = out_type == TG_FP32 ? 0 : 1, dd = head_dim == 64 ? 0 : 1;
  const AttnFn fn = kAttn[io][oo][dd];
  const uint32_t lds = lds_bytes((int)head_dim);
  if (lds > 64 * 1024) {
    if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return TG_ERR_HIP;
  }
  // one work-group per (head, row block); beyond 2^30 items each loops, with
  // a stride that is a multiple of 8 (the XCD order the kernel assumes)
  const int64_t cap = (int64_t)1 << 30;
  const dim3 grid((unsigned)(total < cap ? total : cap), 1);
  hipLaunchKernelGGL(fn, grid, dim3(64 * kWaves), (size_t)lds, stream, a);
  return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // extern "C"
