/*
 * tgemm.h -- tiled bf16/fp16 GEMM and batched GEMM for AMD Instinct MI355X (gfx950).
 *
 * Operation (row-major storage throughout):
 *     C[b] = op(A[b]) * op(B[b])        b = 0 .. batch-1
 * op(X) is X or its transpose.  The product of op(A) (M x K) and op(B) (K x N)
 * is the dense matrix multiply whose 2*M*N*K flops and
 * 2*(M*K + K*N + M*N)-byte footprint the page "Optimize Triton Block
 * Parameters" (Step 1) uses to place a kernel on the roofline.  A transpose is
 * expressed only through the addresses used to read the stored operand
 * ("Triton Optimization Reference", section 2); the batch index only offsets
 * each operand by its own batch stride (same page, section 3).  Inputs are
 * bf16 or fp16, products are accumulated in fp32, and the fp32 sum is written
 * as fp32 or rounded to the input type (round to nearest, ties to even).  C is
 * overwritten, or, through gemm_run_ex/bmm_run_ex, combined with its prior
 * contents by an alpha/beta/bias epilogue.
 *
 * Storage and leading dimensions (all in elements, all row-major):
 *   trans_a = 0: A is M x K, element (i,k) at A[i*lda + k],  lda >= max(1, K)
 *   trans_a = 1: A is stored K x M, op(A)(i,k) = A[k*lda + i], lda >= max(1, M)
 *   trans_b = 0: B is K x N, element (k,j) at B[k*ldb + j],  ldb >= max(1, N)
 *   trans_b = 1: B is stored N x K, op(B)(k,j) = B[j*ldb + k], ldb >= max(1, K)
 *   C is M x N, element (i,j) at C[i*ldc + j],               ldc >= max(1, N)
 * In batched calls the operands of batch b start at A + b*stride_a,
 * B + b*stride_b and C + b*stride_c (elements; a stride of 0 reuses one
 * operand for every batch; C strides must not make batches overlap).
 *
 * Ownership: every pointer is caller-owned device memory (A, B, C) or
 * caller-owned host memory (the plan).  The library allocates nothing and is
 * safe to call from several host threads.  Its only process state is a
 * per-device cache of the compute-unit count and, for
 * gemm_splitk_run_noalloc, one fixed scratch array per device (see there).
 * C must not alias A or B.
 *
 * Errors are returned as tg_status codes; the library never aborts or throws.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_ABI_VERSION 1

typedef enum { TG_BF16 = 0, TG_FP16 = 1, TG_FP32 = 2 } tg_dtype;

typedef enum {
  TG_OK = 0,
  TG_ERR_INVALID = 1,     /* bad argument: sizes, leading dims, flags, null pointers, plan */
  TG_ERR_UNSUPPORTED = 2, /* well-formed but not provided: dtype pair, forced variant/tile */
  TG_ERR_HIP = 3,         /* the HIP runtime rejected the launch */
  TG_ERR_TOO_LARGE = 4    /* the problem needs more scratch than the library's fixed array holds */
} tg_status;

/* Kernel families a plan can select. */
typedef enum {
  TG_VARIANT_GENERIC = 0, /* element-wise loads: any alignment and leading dimension */
  TG_VARIANT_TILE = 1,    /* 16-byte vector loads along each operand's contiguous dim */
  TG_VARIANT_SKINNY = 2   /* M <= 32, both operands K-contiguous: streams B once */
} tg_variant;

/* Entries of the TG_VARIANT_TILE table served by the ping-pong kernel: 8
 * waves in two groups that take turns between a matrix-core phase and a
 * memory phase (256 x 256 tiles, 64-deep K steps, three A and two B LDS
 * buffers, so lds_bytes = (3*bm*bk + 2*bk*bn) * 2).  gemm_plan picks it for
 * large MFMA-bound problems.  TG_TILE_PINGPONG_EPI is the same kernel with the
 * alpha/beta/bias epilogue compiled in; the run calls use whichever of the two
 * matches the call (with or without an epilogue), and the 8-wave tile kernel
 * (entry 3) when K = 0. */
#define TG_TILE_PINGPONG 8
#define TG_TILE_PINGPONG_EPI 9

/* Entry of the TG_VARIANT_TILE table served by the panel kernel, for products
 * with a short K whose time goes into writing C ("Triton Optimization
 * Reference", section 7: persistent programs looping over tiles).  Each
 * work-group walks a run of 128 x 128 tiles along one row panel of C, with A's
 * 128 x K panel held in registers and B's tiles in two LDS buffers, so
 * lds_bytes = 2 * bk * bn * 2 with bk = 128, the largest K it takes.  It
 * serves A stored M x K, 0 < K <= 128, N a multiple of 16 bytes' worth of
 * output elements, and no epilogue.  The run calls send any other call
 * planned on this entry to the 128 x 128 tile kernel (entry 4). */
#define TG_TILE_PANEL 10

/* Entry of the TG_VARIANT_TILE table served by the K-slice kernel, for small
 * products with at most one 64 x 64 tile per CU ("Triton Optimization
 * Reference", section 7: split-K for tiles too few to fill the machine).  The
 * four waves of a work-group each walk a quarter of the tile's K steps (32
 * deep) through a four-stage LDS ring of their own, then sum their partial
 * tiles through LDS; lds_bytes = 4 * stages * (bm*bk + bk*bn) * 2.  Every
 * transpose, epilogue and K (K = 0 included) is served. */
#define TG_TILE_KSLICE 12

/* plan.flags bits */
#define TG_FLAG_EVEN_K 0x1 /* K is a multiple of the K-tile: no masked K step */
#define TG_FLAG_VEC16 0x2  /* leading dims and contiguous extents allow 16-byte loads */
#define TG_FLAG_ROTATE_K 0x4 /* tile kernel: work-groups start their K walks at different steps */
#define TG_FLAG_PERSIST 0x8  /* tile kernel: when there are more tiles than resident work-groups,
                                launch one work-group per resident slot and let each loop over
                                tiles (no dispatch gap between tiles) */
#define TG_FLAG_PREFETCH 0x10 /* with PERSIST: issue the next tile's first copies before this
                                 tile's stores (stores go straight from registers). */
#define TG_FLAG_STREAM_C 0x20 /* tile kernel: store C non-temporally (outputs much larger than the
                                 L2s: the stream of C then does not evict the operands).  A caller
                                 may clear or set PERSIST, PREFETCH, ROTATE_K or STREAM_C in a plan;
                                 the result is the same up to fp32 summation order. */

/*
 * A plan: caller-owned plain data, filled by gemm_plan(), read by gemm_run()
 * and bmm_run().  No heap memory behind it and nothing to destroy.  A caller
 * may overwrite `variant` and `tile` with another supported pair (every pair
 * gives the same result up to fp32 summation order); the run calls validate
 * the pair against the problem and return TG_ERR_UNSUPPORTED if it does not fit.
 */
typedef struct {
  int32_t abi_version;          /* TG_ABI_VERSION, set by gemm_plan */
  int32_t in_type, out_type;    /* tg_dtype */
  int32_t trans_a, trans_b;     /* 0 or 1 */
  int64_t m, n, k, lda, ldb, ldc;
  int32_t variant;              /* tg_variant */
  int32_t tile;                 /* index into the variant's tile table */
  int32_t bm, bn, bk;           /* tile shape of (variant, tile), informational */
  int32_t wg_threads;           /* work-group size */
  int32_t stages;               /* LDS buffers in the K pipeline */
  int32_t flags;                /* TG_FLAG_* */
  uint32_t lds_bytes;           /* LDS per work-group: stages*(bm*bk + bk*bn)*2 */
  uint32_t reserved0;
  uint64_t workspace_bytes;     /* always 0: no workspace */
  int64_t tiles_m, tiles_n;     /* work-groups per matrix = tiles_m * tiles_n */
} gemm_plan_t;

/*
 * gemm_plan -- validate a problem and choose kernel and tile.  Host only: no
 * device call, no allocation.
 *   in_type : TG_BF16 or TG_FP16 (A and B alike)
 *   out_type: TG_FP32, or the same type as in_type
 *   m, n, k >= 0; leading dims as in the table above.
 * Returns TG_OK, TG_ERR_INVALID (null plan, negative size, trans not 0/1,
 * leading dim too small, size product overflow) or TG_ERR_UNSUPPORTED
 * (dtype pair).  Tile choice follows the shape: M <= 32 with both operands
 * K-contiguous selects the skinny kernel; otherwise the tile is sized so that
 * the grid covers the chip, and the 16-byte vector loader is chosen when
 * every leading dimension and every operand's contiguous extent is a
 * multiple of 8 elements.
 */
tg_status gemm_plan(gemm_plan_t* plan, tg_dtype in_type, tg_dtype out_type, int trans_a, int trans_b,
                    int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb, int64_t ldc);

/*
 * bmm_plan -- gemm_plan for a batch of `batch` >= 1 products of the same
 * shape (run with bmm_run): the tile choice counts work items over the whole
 * batch.  gemm_plan(...) is bmm_plan(..., 1).  Same errors as gemm_plan, plus
 * TG_ERR_INVALID for batch < 1.  Any valid plan may be passed to bmm_run with
 * any batch count; this one is tuned for the count given here.
 */
tg_status bmm_plan(gemm_plan_t* plan, tg_dtype in_type, tg_dtype out_type, int trans_a, int trans_b,
                   int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb, int64_t ldc, int64_t batch);

/*
 * gemm_plan_tile -- re-plan a valid plan for a caller-chosen kernel variant
 * (tg_variant) and tile index (0 .. tg_variant_tiles(variant)-1): fills the
 * same derived fields gemm_plan fills (bm, bn, bk, wg_threads, stages, flags,
 * lds_bytes, tiles_m, tiles_n) for that choice.  Returns TG_ERR_INVALID for a
 * null or stale plan and TG_ERR_UNSUPPORTED for a variant/tile that cannot
 * run this problem; the plan is left unchanged on error.  Every choice gives
 * the same result up to the order of fp32 additions.
 */
tg_status gemm_plan_tile(gemm_plan_t* plan, int32_t variant, int32_t tile);

/*
 * gemm_run -- enqueue C = op(A) op(B) on `stream` (0 = the null stream) and
 * return without waiting.  A, B, C are device pointers.  If the plan chose the
 * vector loader but a base pointer is not 16-byte aligned, the element-wise
 * loader runs instead (same result).  M = 0 or N = 0 launches nothing; K = 0
 * writes zeros to C.  Returns TG_ERR_INVALID for a null or stale plan
 * (abi_version) or a null pointer with a nonzero extent, TG_ERR_UNSUPPORTED
 * for a (variant, tile) pair that does not fit the problem, TG_ERR_HIP if the
 * launch fails.
 */
tg_status gemm_run(const gemm_plan_t* plan, const void* A, const void* B, void* C, hipStream_t stream);

/*
 * bmm_run -- batched form: batch >= 0 independent products, operand b at
 * A + b*stride_a, B + b*stride_b, C + b*stride_c (elements, >= 0; byte offsets
 * are 64-bit).  batch = 0 launches nothing.  Same errors as gemm_run, plus
 * TG_ERR_INVALID for a negative batch or stride.
 */
tg_status bmm_run(const gemm_plan_t* plan, int64_t batch, int64_t stride_a, int64_t stride_b,
                  int64_t stride_c, const void* A, const void* B, void* C, hipStream_t stream);

/*
 * gemm_group_run -- many independent products of different shapes in as few
 * launches as possible: C_i = op(A_i) op(B_i), i = 0 .. count-1, all with the
 * same types and transposes.  It applies the pages' batched-launch idea
 * ("Triton Optimization Reference", section 8: several tensors per launch,
 * with the host grouping them, to pay the launch overhead once) to GEMM
 * lists: up to TG_GROUP_MAX problems share one grid, each work-group looking
 * its problem up in a table passed with the launch arguments.
 *   problems: caller-owned host array of `count` >= 0 descriptors (read
 *     during the call only); each descriptor's sizes and leading dimensions
 *     follow the storage table above; A, B, C are device pointers.
 *   tile: -1 lets the library choose one tile shape per launch from the
 *     group's totals; 0 .. tg_group_tiles()-1 forces one (tests, tuning).
 * Problems with m = 0 or n = 0 are skipped; k = 0 writes zeros.  Problems the
 * 16-byte vector loader cannot serve (misaligned base, leading dim or
 * contiguous extent not a multiple of 8) run one by one through the
 * element-wise loader.  Every problem is validated before anything is
 * enqueued.  C_i must not alias any A_j, B_j or another C_j.  The library
 * allocates nothing.  Returns TG_OK, TG_ERR_INVALID (count < 0, null array,
 * an invalid problem as gemm_plan defines it, a null pointer with nonzero
 * extents, more than 2^30 tiles in a problem), TG_ERR_UNSUPPORTED (dtype
 * pair, tile out of range), TG_ERR_HIP.
 */
#define TG_GROUP_MAX 32

typedef struct {
  int64_t m, n, k;
  int64_t lda, ldb, ldc;
  const void* A;
  const void* B;
  void* C;
} gemm_group_problem_t;

tg_status gemm_group_run(tg_dtype in_type, tg_dtype out_type, int trans_a, int trans_b,
                         const gemm_group_problem_t* problems, int64_t count, int32_t tile, hipStream_t stream);

/* Number of tile shapes a grouped launch can be forced to (gemm_group_run's `tile`). */
int32_t tg_group_tiles(void);

/*
 * gemm_splitk_run -- the product a plan describes, C = op(A) op(B), with K
 * cut into parts: for shapes whose output tiles are too few to occupy the
 * chip while K is long ("Triton Optimization Reference", section 7: the
 * persistent / stream-K family of schedules, for when the tile grid alone
 * leaves compute units idle).  Part s covers k in [s*ks, min(K, (s+1)*ks)),
 * ks = ceil(K / splits) rounded up to a multiple of 8, so there are
 * ceil(K / ks) <= splits parts.  Enqueued on `stream`:
 *   1. the parts of exactly ks as one batched product (bmm_plan + bmm_run,
 *      the batch strides stepping along K), each into fp32 slice s of
 *      `workspace`, which is laid out as parts x m rows of ldw = n rounded
 *      up to 8 floats; a shorter last part as one more product (gemm_plan +
 *      gemm_run) into the last slice;
 *   2. a reduction that adds the slices in a fixed order (slice 0 first) and
 *      writes C in the plan's output type (nearest-even for 16-bit outputs).
 * The result is deterministic.  It equals gemm_run's up to the order of
 * fp32 additions, and bit for bit where every partial sum is exact.  The
 * plan's variant and tile are not used (the parts are planned for their own
 * shape); its types, transposes, sizes and leading dimensions are.
 *   splits: 1 .. TG_SPLITK_MAX (tg_splitk_choose suggests one).
 *   workspace: caller-owned device memory of at least
 *     tg_splitk_workspace_bytes(plan, splits) bytes, 16-byte aligned; it is
 *     fully overwritten where used, and must not overlap A, B or C.  It is
 *     in use until the work on `stream` completes.  It may be null when
 *     K = 0 (then C is zeroed).
 *   A, B, C: device pointers as for gemm_run; C naturally aligned.
 * The library allocates nothing.  Returns TG_OK (m = 0 or n = 0: nothing
 * enqueued), TG_ERR_INVALID (null or stale plan, splits out of range, a
 * null pointer with nonzero extents, a workspace too small or misaligned),
 * TG_ERR_UNSUPPORTED or TG_ERR_HIP as bmm_run does.  All checks run before
 * anything is enqueued.
 */
#define TG_SPLITK_MAX 32
tg_status gemm_splitk_run(const gemm_plan_t* plan, int32_t splits, void* workspace, uint64_t workspace_bytes,
                          const void* A, const void* B, void* C, hipStream_t stream);

/*
 * gemm_splitk_run_noalloc -- gemm_splitk_run without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The partial
 * products go to a fixed array of TG_SPLITK_SCRATCH_BYTES in device memory
 * that the library holds once per GPU until the process ends; its device
 * address is looked up on the first call on each device (with that device
 * current).  Nothing is allocated and no allocating routine is called.
 *   Same arguments, results and errors as gemm_splitk_run (the parts, the
 *   reduction and the order of additions are the same, so the results are
 *   bit-identical), plus TG_ERR_TOO_LARGE when
 *   tg_splitk_workspace_bytes(plan, splits) > TG_SPLITK_SCRATCH_BYTES
 *   (checked before any device call), and TG_ERR_HIP if the device or the
 *   array's address cannot be obtained.
 *   Every call on one GPU uses that GPU's one array, and the array keeps the
 *   last call's partial products: calls that may overlap on one GPU (several
 *   streams, or several host threads, at once) race and give wrong results;
 *   serialise them (one stream, or events between them).  The reduction reads
 *   only what the parts of the same call wrote, so nothing has to start at
 *   zero.
 */
#define TG_SPLITK_SCRATCH_BYTES (64ull << 20)
tg_status gemm_splitk_run_noalloc(const gemm_plan_t* plan, int32_t splits, const void* A, const void* B, void* C,
                                  hipStream_t stream);

/* Workspace bytes gemm_splitk_run needs for `plan` and `splits`
 * (parts * m * ldw * 4); 0 for an invalid plan or split count, or K = 0. */
uint64_t tg_splitk_workspace_bytes(const gemm_plan_t* plan, int32_t splits);

/* A split count for `plan`, counted in output tiles of 256 x 256 (the
 * ping-pong kernel's).  1 (do not split) when the product has 128 or more of
 * them or K < 2048.  Otherwise the most parts that fit one round of MI355X's
 * 256 CUs with parts at least 2048 deep, if that makes 144 or more work
 * items; else, for outputs of at most 16 such tiles, enough parts for 256
 * items with parts at least 512 deep; else 1.  At most TG_SPLITK_MAX.
 * Host-only; 1 for an invalid plan. */
int32_t tg_splitk_choose(const gemm_plan_t* plan);

/*
 * attention_fwd -- fused attention forward pass, enqueued on `stream`:
 *     O[b] = softmax(scale * Q[b] K[b]^T) V[b]        b = 0 .. batch-1
 * the attention-shaped pair of products the pages' GEMM/BMM/attention
 * reference names as its companion target ("Triton Optimization Reference
 * (cuTile -> Triton)", opening section), chained through a row softmax
 * (over all n_k keys: no mask) inside one kernel, so the n_q x n_k scores
 * and probabilities never reach memory.
 *   Q[b] is n_q x head_dim, element (i,c) at Q + b*stride_q + i*ldq + c;
 *   K[b] and V[b] are n_k x head_dim, likewise with ldk/stride_k, ldv/stride_v;
 *   O[b] is n_q x head_dim at O + b*stride_o + i*ldo + c   (all in elements).
 * in_type: TG_BF16 or TG_FP16 (Q, K, V alike); out_type: TG_FP32 or in_type.
 * Scores and sums are fp32; the probabilities are rounded to in_type before
 * the product with V (round to nearest even), and O to out_type.
 * head_dim: 64 or 128.  scale: finite and > 0 (1/sqrt(head_dim) is the usual
 * choice).  Leading dims >= head_dim, < 2^20, multiples of 8; the four base
 * pointers 16-byte aligned and (batch > 1) the strides multiples of 8; each
 * head's K and V span under 2 GiB ((n_k - 1) * ld + head_dim < 2^30 elements).
 * Ownership: all pointers are caller-owned device memory; nothing is
 * allocated.  O must not alias Q, K or V; heads' outputs must not overlap.
 * Returns TG_OK (batch = 0 or n_q = 0 launches nothing), TG_ERR_INVALID
 * (negative size or stride, n_k = 0 with work to do, bad scale, leading dim
 * below head_dim, null pointer, overlapping outputs, offset overflow),
 * TG_ERR_UNSUPPORTED (dtype pair, head_dim, alignment, leading dim >= 2^20,
 * a head's K or V span of 2 GiB or more),
 * TG_ERR_HIP (launch failed).
 */
tg_status attention_fwd(tg_dtype in_type, tg_dtype out_type, int64_t batch, int64_t n_q, int64_t n_k,
                        int64_t head_dim, float scale, const void* Q, int64_t ldq, int64_t stride_q,
                        const void* K, int64_t ldk, int64_t stride_k, const void* V, int64_t ldv,
                        int64_t stride_v, void* O, int64_t ldo, int64_t stride_o, hipStream_t stream);

/*
 * Optional epilogue of gemm_run_ex / bmm_run_ex, applied to the fp32 sum
 * before the output rounding:
 *     C = alpha * op(A) op(B) + beta * C + bias[j]
 * (the scaled-and-shifted product the pages count as a trivial epilogue:
 * "Finetuning Your Program", the alpha/beta note).  C's prior contents are
 * read only when beta != 0 (with beta = 0, NaN or Inf in C are ignored, as
 * in BLAS).  bias: null, or a device array of n values of the output type
 * (fp32 for an fp32 output, else the input type), naturally aligned, added to
 * every row (and, in a batch, to every matrix).  alpha = 1, beta = 0 and no
 * bias is exactly the plain product.
 */
typedef struct {
  float alpha;
  float beta;
  const void* bias;
} gemm_epilogue_t;

/*
 * gemm_run_ex / bmm_run_ex -- gemm_run / bmm_run with an epilogue (null: none).
 * Same errors, plus TG_ERR_INVALID for a misaligned bias.  With an epilogue
 * the persistent launch modes (TG_FLAG_PERSIST, TG_FLAG_PREFETCH) are not
 * used; the result does not depend on them.
 */
tg_status gemm_run_ex(const gemm_plan_t* plan, const gemm_epilogue_t* epi, const void* A, const void* B, void* C,
                      hipStream_t stream);
tg_status bmm_run_ex(const gemm_plan_t* plan, const gemm_epilogue_t* epi, int64_t batch, int64_t stride_a,
                     int64_t stride_b, int64_t stride_c, const void* A, const void* B, void* C, hipStream_t stream);

/* Static text for a status code ("ok", "invalid argument", ...). */
const char* tg_status_str(tg_status s);

/* TG_ABI_VERSION of the built library, to detect a header/library mismatch. */
int32_t tg_abi_version(void);

/*
 * Number of tile shapes the library holds for `variant` (one of tg_variant);
 * valid `tile` values in a caller-overridden plan are 0 .. count-1.  Returns
 * 0 for an unknown variant.  Every shape yields the same result up to the
 * order of fp32 additions (for integer-valued inputs, bit-identical).
 */
int32_t tg_variant_tiles(int32_t variant);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
