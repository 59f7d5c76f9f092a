// splitk.hip -- split-K products: C = op(A) op(B) with K cut into parts that
// run as independent products, for shapes with too few output tiles to fill
// the chip and a long K ("Triton Optimization Reference", section 7: the
// persistent / stream-K family of schedules for when the tile grid alone
// leaves compute units idle).
//
// The parts of equal length go out as one batched product (bmm_plan +
// bmm_run: part s reads A's and B's K range [s*ks, (s+1)*ks) through batch
// strides and writes fp32 slice s of the caller's workspace), a shorter last
// part as one more product, and one reduction kernel adds the slices in a
// fixed order (slice 0 first) and writes C in the output type.  The batched
// product gets the planner's kernel for its shape -- the ping-pong kernel
// once the parts make more than 128 of its 256x256 work items.  Every launch
// goes on the caller's stream; the library allocates nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/tgemm.h"

// Partial products of gemm_splitk_run_noalloc: a fixed array in device
// memory, one copy per GPU the library runs on, held until the process ends.
// Host code never passes this name to a kernel (on the host it only stands in
// for the symbol); it asks the runtime for each device's address once and
// uses that.
static __device__ __align__(256) float scratch[TG_SPLITK_SCRATCH_BYTES / sizeof(float)];

namespace {

// Device address of `scratch` on each device, filled on the first
// gemm_splitk_run_noalloc call on that device (racing fills store the same
// value).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

tg_status scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TG_ERR_UNSUPPORTED;
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TG_ERR_HIP;
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
  }
  *out = static_cast<float*>(ptr);
  return TG_OK;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Part geometry: ks k-elements per part (a multiple of 8, so every part's A
// and B bases stay 16-byte aligned), `parts` parts (the last may be
// shorter), workspace rows of ldw = N rounded up to 8 floats.
struct Parts {
  int64_t ks, parts, ldw;
};
Parts parts_of(const gemm_plan_t& p, int32_t splits) {
  Parts r;
  r.ks = p.k > 0 ? round_up(cdiv(p.k, splits), 8) : 0;
  r.parts = p.k > 0 ? cdiv(p.k, r.ks) : 0;
  r.ldw = round_up(p.n > 0 ? p.n : 1, 8);
  return r;
}

// C[i][j] = sum over parts s (in order) of W[s][i][j], rounded to Out.
// Thread q handles 4 consecutive columns of one row: one 16-byte load per
// part (ldw and the slice stride are multiples of 4 floats, so the loads are
// aligned; columns N .. ldw-1 are read but never stored).
template <typename Out>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ W, int64_t slice, int32_t parts,
                                                            int64_t M, int64_t N, int64_t ldw, Out* __restrict__ C,
                                                            int64_t ldc) {
  const int64_t groups = (N + 3) / 4;
  const int64_t total = M * groups;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int64_t i = q / groups, j = (q - i * groups) * 4;
    const float* w = W + i * ldw + j;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int32_t p = 0; p < parts; ++p) {
      const f32x4 v = *(const f32x4*)(w + p * slice);
      s[0] += v[0];
      s[1] += v[1];
      s[2] += v[2];
      s[3] += v[3];
    }
    Out* c = C + i * ldc + j;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e < N) c[e] = (Out)s[e];  // nearest, ties to even, for 16-bit outputs
  }
}

}  // namespace

extern "C" {

uint64_t tg_splitk_workspace_bytes(const gemm_plan_t* plan, int32_t splits) {
  if (!plan || plan->abi_version != TG_ABI_VERSION || splits < 1 || splits > TG_SPLITK_MAX) return 0;
  const Parts g = parts_of(*plan, splits);
  const double bytes = 4.0 * (double)g.parts * (double)plan->m * (double)g.ldw;
  if (bytes >= 4.0e18) return 0;
  return (uint64_t)g.parts * (uint64_t)plan->m * (uint64_t)g.ldw * 4u;
}

int32_t tg_splitk_choose(const gemm_plan_t* plan) {
  if (!plan || plan->abi_version != TG_ABI_VERSION) return 1;
  const gemm_plan_t& p = *plan;
  // Counted in 256 x 256 tiles (the ping-pong kernel's): a product with 128
  // or more of them already runs on that kernel whole.  Otherwise one round
  // of work items on MI355X's 256 CUs with parts at least 2048 deep, if that
  // gives 144 or more items (with fewer, the plain launch's smaller tiles
  // measured as fast); tiny outputs (<= 16 such tiles, which a plain launch
  // leaves almost serial) split further, down to parts of 512.
  const int64_t tiles = cdiv(p.m, 256) * cdiv(p.n, 256);
  if (tiles == 0 || tiles >= 128 || p.k < 2048) return 1;
  int64_t s = 256 / tiles;
  if (s > p.k / 2048) s = p.k / 2048;
  if (s > TG_SPLITK_MAX) s = TG_SPLITK_MAX;
  if (s >= 2 && tiles * s >= 144) return (int32_t)s;
  if (tiles > 16) return 1;
  s = cdiv(256, tiles);
  if (s > p.k / 512) s = p.k / 512;
  if (s > TG_SPLITK_MAX) s = TG_SPLITK_MAX;
  return (int32_t)(s < 1 ? 1 : s);
}

}  // extern "C"

namespace {

// Checks shared by both entry points (everything but the workspace).
tg_status splitk_check(const gemm_plan_t* plan, int32_t splits, const void* A, const void* B, const void* C) {
  if (!plan || plan->abi_version != TG_ABI_VERSION) return TG_ERR_INVALID;
  if (splits < 1 || splits > TG_SPLITK_MAX) return TG_ERR_INVALID;
  const gemm_plan_t& p = *plan;
  if (p.in_type < 0 || p.in_type > 1 || (p.out_type != TG_FP32 && p.out_type != p.in_type)) return TG_ERR_INVALID;
  if (p.m == 0 || p.n == 0) return TG_OK;
  if (!C) return TG_ERR_INVALID;
  if (p.k > 0 && (!A || !B)) return TG_ERR_INVALID;
  if (p.k > 0 && tg_splitk_workspace_bytes(plan, splits) == 0) return TG_ERR_INVALID;
  return TG_OK;
}

// Enqueue the parts into the fp32 workspace W (large enough, 16-byte
// aligned, checked by the caller) and the reduction into C.
tg_status splitk_enqueue(const gemm_plan_t& p, int32_t splits, float* W, const void* A, const void* B, void* C,
                         hipStream_t stream) {
  const Parts g = parts_of(p, splits);
  const int64_t slice = p.m * g.ldw;  // floats per part
  const char* a = static_cast<const char*>(A);
  const char* b = static_cast<const char*>(B);
  // K runs along A's rows when A is stored M x K, down its rows when stored
  // K x M; likewise B (along its rows when stored N x K)
  auto a_at = [&](int64_t k0) { return a + 2 * (p.trans_a ? k0 * p.lda : k0); };
  auto b_at = [&](int64_t k0) { return b + 2 * (p.trans_b ? k0 : k0 * p.ldb); };
  const tg_dtype in = (tg_dtype)p.in_type;
  const int64_t full = g.ks > 0 ? p.k / g.ks : 0;  // parts of exactly ks (none when K = 0)
  const int64_t tail = p.k - full * g.ks;           // a shorter last part (0: none)
  // both plans are made (and checked) before anything is enqueued
  gemm_plan_t qf, qt;
  if (full > 0) {
    const tg_status st = bmm_plan(&qf, in, TG_FP32, p.trans_a, p.trans_b, p.m, p.n, g.ks, p.lda, p.ldb, g.ldw, full);
    if (st != TG_OK) return st;
  }
  if (tail > 0) {
    const tg_status st = gemm_plan(&qt, in, TG_FP32, p.trans_a, p.trans_b, p.m, p.n, tail, p.lda, p.ldb, g.ldw);
    if (st != TG_OK) return st;
  }
  if (full > 0) {
    const int64_t sa = p.trans_a ? g.ks * p.lda : g.ks, sb = p.trans_b ? g.ks : g.ks * p.ldb;
    const tg_status st = bmm_run(&qf, full, sa, sb, slice, a, b, W, stream);
    if (st != TG_OK) return st;
  }
  if (tail > 0) {
    const tg_status st = gemm_run(&qt, a_at(full * g.ks), b_at(full * g.ks), W + full * slice, stream);
    if (st != TG_OK) return st;
  }
  const int64_t total = p.m * cdiv(p.n, 4);
  const int64_t blocks64 = cdiv(total, 256);
  const unsigned blocks = (unsigned)(blocks64 < 8192 ? blocks64 : 8192);
  const int32_t parts = (int32_t)g.parts;
  if (p.out_type == TG_FP32)
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(blocks), dim3(256), 0, stream, W, slice, parts, p.m, p.n,
                       g.ldw, static_cast<float*>(C), p.ldc);
  else if (p.out_type == TG_BF16)
    hipLaunchKernelGGL(splitk_reduce_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream, W, slice, parts, p.m, p.n,
                       g.ldw, static_cast<__bf16*>(C), p.ldc);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<_Float16>, dim3(blocks), dim3(256), 0, stream, W, slice, parts, p.m,
                       p.n, g.ldw, static_cast<_Float16*>(C), p.ldc);
  return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace

extern "C" {

tg_status gemm_splitk_run(const gemm_plan_t* plan, int32_t splits, void* workspace, uint64_t workspace_bytes,
                          const void* A, const void* B, void* C, hipStream_t stream) {
  const tg_status st = splitk_check(plan, splits, A, B, C);
  if (st != TG_OK || plan->m == 0 || plan->n == 0) return st;
  const uint64_t need = tg_splitk_workspace_bytes(plan, splits);
  if (plan->k > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 16 != 0)) return TG_ERR_INVALID;
  return splitk_enqueue(*plan, splits, static_cast<float*>(workspace), A, B, C, stream);
}

tg_status gemm_splitk_run_noalloc(const gemm_plan_t* plan, int32_t splits, const void* A, const void* B, void* C,
                                  hipStream_t stream) {
  const tg_status st = splitk_check(plan, splits, A, B, C);
  if (st != TG_OK || plan->m == 0 || plan->n == 0) return st;
  if (tg_splitk_workspace_bytes(plan, splits) > TG_SPLITK_SCRATCH_BYTES) return TG_ERR_TOO_LARGE;
  float* W = nullptr;
  const tg_status sw = scratch_of_current_device(&W);
  if (sw != TG_OK) return sw;
  return splitk_enqueue(*plan, splits, W, A, B, C, stream);
}

}  // extern "C"
