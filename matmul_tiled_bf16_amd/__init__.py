"""Tiled bf16/fp16 GEMM and batched GEMM for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libtgemm.so`` (``include/tgemm.h``): argument
marshalling only -- every arithmetic step runs in the library's HIP kernels,
and there is no fallback.  If the library is not built, every call raises.

    import torch, matmul_tiled_bf16_amd as tg
    C = tg.gemm(A, B, trans_b=True, out_dtype=torch.bfloat16)   # C = A @ B^T

Matrices are row-major torch tensors whose last dimension is contiguous; a
transpose is requested with ``trans_a``/``trans_b`` and is never materialised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtgemm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "tgemm.h")

TG_BF16, TG_FP16, TG_FP32 = 0, 1, 2
TG_OK, TG_ERR_INVALID, TG_ERR_UNSUPPORTED, TG_ERR_HIP, TG_ERR_TOO_LARGE = 0, 1, 2, 3, 4
VARIANT_GENERIC, VARIANT_TILE, VARIANT_SKINNY = 0, 1, 2
TILE_PINGPONG, TILE_PINGPONG_EPI = 8, 9  # TG_TILE_PINGPONG, TG_TILE_PINGPONG_EPI
TILE_PANEL = 10  # TG_TILE_PANEL
TILE_KSLICE = 12  # TG_TILE_KSLICE
SPLITK_MAX = 32  # TG_SPLITK_MAX
SPLITK_SCRATCH_BYTES = 64 << 20  # TG_SPLITK_SCRATCH_BYTES
FLAG_EVEN_K, FLAG_VEC16, FLAG_ROTATE_K, FLAG_PERSIST, FLAG_PREFETCH, FLAG_STREAM_C = 0x1, 0x2, 0x4, 0x8, 0x10, 0x20


def _abi_version_from_header() -> int:
    with open(HEADER) as f:
        m = re.search(r"#define\s+TG_ABI_VERSION\s+(\d+)", f.read())
    return int(m.group(1))


class GemmPlan(ctypes.Structure):
    """Mirror of gemm_plan_t."""
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("in_type", ctypes.c_int32), ("out_type", ctypes.c_int32),
        ("trans_a", ctypes.c_int32), ("trans_b", ctypes.c_int32),
        ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
        ("variant", ctypes.c_int32), ("tile", ctypes.c_int32),
        ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
        ("wg_threads", ctypes.c_int32), ("stages", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("lds_bytes", ctypes.c_uint32), ("reserved0", ctypes.c_uint32),
        ("workspace_bytes", ctypes.c_uint64),
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
    ]

    def __repr__(self):
        return ("GemmPlan(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_
                                         if n != "reserved0") + ")")


class GroupProblem(ctypes.Structure):
    """Mirror of gemm_group_problem_t."""
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p)]


class Epilogue(ctypes.Structure):
    """Mirror of gemm_epilogue_t: C = alpha * op(A) op(B) + beta * C + bias[j]."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("bias", ctypes.c_void_p)]


class TgError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m matmul_tiled_bf16_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.gemm_plan.restype = ctypes.c_int
        L.gemm_plan.argtypes = [ctypes.POINTER(GemmPlan), ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                i64, i64, i64, i64, i64, i64]
        L.gemm_run.restype = ctypes.c_int
        L.gemm_run.argtypes = [ctypes.POINTER(GemmPlan), p, p, p, p]
        L.bmm_run.restype = ctypes.c_int
        L.bmm_run.argtypes = [ctypes.POINTER(GemmPlan), i64, i64, i64, i64, p, p, p, p]
        L.tg_status_str.restype = ctypes.c_char_p
        L.tg_status_str.argtypes = [ctypes.c_int]
        L.tg_abi_version.restype = i32
        L.tg_abi_version.argtypes = []
        L.tg_variant_tiles.restype = i32
        L.tg_variant_tiles.argtypes = [i32]
        L.bmm_plan.restype = ctypes.c_int
        L.bmm_plan.argtypes = [ctypes.POINTER(GemmPlan), ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               i64, i64, i64, i64, i64, i64, i64]
        L.gemm_plan_tile.restype = ctypes.c_int
        L.gemm_plan_tile.argtypes = [ctypes.POINTER(GemmPlan), i32, i32]
        L.gemm_run_ex.restype = ctypes.c_int
        L.gemm_run_ex.argtypes = [ctypes.POINTER(GemmPlan), ctypes.POINTER(Epilogue), p, p, p, p]
        L.bmm_run_ex.restype = ctypes.c_int
        L.bmm_run_ex.argtypes = [ctypes.POINTER(GemmPlan), ctypes.POINTER(Epilogue), i64, i64, i64, i64, p, p, p, p]
        L.gemm_group_run.restype = ctypes.c_int
        L.gemm_group_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(GroupProblem), i64, i32, p]
        L.tg_group_tiles.restype = i32
        L.tg_group_tiles.argtypes = []
        L.gemm_splitk_run.restype = ctypes.c_int
        L.gemm_splitk_run.argtypes = [ctypes.POINTER(GemmPlan), i32, p, ctypes.c_uint64, p, p, p, p]
        L.gemm_splitk_run_noalloc.restype = ctypes.c_int
        L.gemm_splitk_run_noalloc.argtypes = [ctypes.POINTER(GemmPlan), i32, p, p, p, p]
        L.tg_splitk_workspace_bytes.restype = ctypes.c_uint64
        L.tg_splitk_workspace_bytes.argtypes = [ctypes.POINTER(GemmPlan), i32]
        L.tg_splitk_choose.restype = i32
        L.tg_splitk_choose.argtypes = [ctypes.POINTER(GemmPlan)]
        L.attention_fwd.restype = ctypes.c_int
        L.attention_fwd.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, ctypes.c_float,
                                    p, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, p]
        if L.tg_abi_version() != _abi_version_from_header():
            raise RuntimeError("libtgemm.so was built from a different tgemm.h (ABI version mismatch)")
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().tg_status_str(int(s)).decode()


def variant_tiles(variant: int) -> int:
    """Number of tile shapes the library holds for `variant` (valid plan.tile values)."""
    return int(lib().tg_variant_tiles(variant))


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.bfloat16:
        return TG_BF16
    if dt == torch.float16:
        return TG_FP16
    if dt == torch.float32:
        return TG_FP32
    raise TypeError(f"unsupported dtype {dt}")


def plan(m: int, n: int, k: int, *, trans_a: bool = False, trans_b: bool = False, in_dtype=None,
         out_dtype=None, lda: Optional[int] = None, ldb: Optional[int] = None,
         ldc: Optional[int] = None, batch: int = 1) -> GemmPlan:
    """bmm_plan() (gemm_plan() for batch 1): validate and choose kernel/tile (host only)."""
    import torch
    in_dtype = torch.bfloat16 if in_dtype is None else in_dtype
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    lda = lda if lda is not None else max(1, m if trans_a else k)
    ldb = ldb if ldb is not None else max(1, k if trans_b else n)
    ldc = ldc if ldc is not None else max(1, n)
    p = GemmPlan()
    st = lib().bmm_plan(ctypes.byref(p), _dtype_code(in_dtype), _dtype_code(out_dtype), int(trans_a),
                        int(trans_b), m, n, k, lda, ldb, ldc, batch)
    if st != TG_OK:
        raise TgError(st, "bmm_plan")
    return p


def plan_tile(p: GemmPlan, variant: int, tile: int) -> GemmPlan:
    """gemm_plan_tile(): a copy of `p` re-planned for the given variant and tile."""
    q = GemmPlan.from_buffer_copy(p)
    st = lib().gemm_plan_tile(ctypes.byref(q), variant, tile)
    if st != TG_OK:
        raise TgError(st, "gemm_plan_tile")
    return q


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    if t is None:
        return None  # a null pointer
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def gemm_run(p: GemmPlan, A, B, C, stream=None) -> None:
    """gemm_run(): enqueue on ``stream`` (torch stream, raw handle, or current)."""
    st = lib().gemm_run(ctypes.byref(p), _ptr(A), _ptr(B), _ptr(C), _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "gemm_run")


def bmm_run(p: GemmPlan, batch: int, stride_a: int, stride_b: int, stride_c: int, A, B, C,
            stream=None) -> None:
    st = lib().bmm_run(ctypes.byref(p), batch, stride_a, stride_b, stride_c, _ptr(A), _ptr(B), _ptr(C),
                       _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "bmm_run")


def _epilogue(alpha, beta, bias):
    if alpha == 1.0 and beta == 0.0 and bias is None:
        return None
    return Epilogue(alpha, beta, _ptr(bias) if bias is not None else None)


def gemm_run_ex(p: GemmPlan, A, B, C, *, alpha: float = 1.0, beta: float = 0.0, bias=None, stream=None) -> None:
    """gemm_run_ex(): C = alpha * op(A) op(B) + beta * C + bias (bias: n values of C's dtype)."""
    e = _epilogue(alpha, beta, bias)
    st = lib().gemm_run_ex(ctypes.byref(p), ctypes.byref(e) if e else None, _ptr(A), _ptr(B), _ptr(C),
                           _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "gemm_run_ex")


def bmm_run_ex(p: GemmPlan, batch: int, stride_a: int, stride_b: int, stride_c: int, A, B, C, *,
               alpha: float = 1.0, beta: float = 0.0, bias=None, stream=None) -> None:
    e = _epilogue(alpha, beta, bias)
    st = lib().bmm_run_ex(ctypes.byref(p), ctypes.byref(e) if e else None, batch, stride_a, stride_b, stride_c,
                          _ptr(A), _ptr(B), _ptr(C), _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "bmm_run_ex")


def _check_matrix(X, name, dims=(2,), out=False):
    """Validate a row-major operand before anything reaches the library.

    The kernels address element (r, c) of a matrix at base + r*ld + c with
    ld = stride(-2), so the last dimension must be contiguous and rows must not
    overlap (stride(-2) >= shape[-1] whenever there are two or more rows);
    otherwise the kernels would read or write outside the tensor's storage.
    A 3-D input may share one matrix across the batch (stride(0) = 0); a 3-D
    output's matrices must not overlap.  Shape checks come first, so they
    raise the same ValueError with or without a GPU."""
    if X.dim() not in dims:
        raise ValueError(f"{name} must be a {' or '.join(f'{d}-D' for d in dims)} tensor, got {X.dim()}-D")
    rows, cols = X.shape[-2], X.shape[-1]
    if cols > 1 and X.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension (stride(-1) = {X.stride(-1)})")
    if rows > 1 and X.stride(-2) < cols:
        raise ValueError(f"{name}: rows overlap (stride(-2) = {X.stride(-2)} < {cols} columns)")
    if out and X.dim() == 3 and X.shape[0] > 1 and rows > 0 and cols > 0:
        span = (rows - 1) * _ld(X) + cols
        if X.stride(0) < span:
            raise ValueError(f"{name}: matrices of the batch overlap (stride(0) = {X.stride(0)} < {span})")
    if not X.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _ld(X) -> int:
    return max(X.stride(-2), X.shape[-1], 1)


def _check_out(out, shape, out_dtype, dims=(2,)):
    if tuple(out.shape) != tuple(shape) or out.dtype != out_dtype:
        raise ValueError(f"out has the wrong shape or dtype: {tuple(out.shape)} {out.dtype}, "
                         f"expected {tuple(shape)} {out_dtype}")
    _check_matrix(out, "out", dims, out=True)


def gemm(A, B, *, trans_a: bool = False, trans_b: bool = False, out_dtype=None, out=None, alpha: float = 1.0,
         beta: float = 0.0, bias=None, stream=None):
    """C = alpha * op(A) @ op(B) + beta * C + bias for 2-D row-major tensors; returns C
    (new, or ``out``, whose prior contents are read when beta != 0)."""
    import torch
    _check_matrix(A, "A")
    _check_matrix(B, "B")
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    m, k = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    kb, n = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
    if kb != k:
        raise ValueError(f"inner dimensions differ: {k} vs {kb}")
    out_dtype = out_dtype or torch.float32
    if beta != 0.0 and out is None:
        raise ValueError("beta != 0 needs `out` (the C to scale)")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=A.device)
    else:
        _check_out(out, (m, n), out_dtype)
    if bias is not None and (bias.dtype != out_dtype or bias.numel() != n or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous tensor of n values of the output dtype")
    p = plan(m, n, k, trans_a=trans_a, trans_b=trans_b, in_dtype=A.dtype, out_dtype=out_dtype, lda=_ld(A),
             ldb=_ld(B), ldc=_ld(out))
    gemm_run_ex(p, A, B, out, alpha=alpha, beta=beta, bias=bias, stream=stream)
    return out


def splitk_workspace_bytes(p: GemmPlan, splits: int) -> int:
    """tg_splitk_workspace_bytes(): bytes of fp32 workspace gemm_splitk_run needs."""
    return int(lib().tg_splitk_workspace_bytes(ctypes.byref(p), int(splits)))


def splitk_choose(p: GemmPlan) -> int:
    """tg_splitk_choose(): a split count for the plan's product (1: do not split)."""
    return int(lib().tg_splitk_choose(ctypes.byref(p)))


def gemm_splitk_run(p: GemmPlan, splits: int, workspace, workspace_bytes: int, A, B, C, stream=None) -> None:
    """gemm_splitk_run(): raw call (pointers or tensors)."""
    st = lib().gemm_splitk_run(ctypes.byref(p), int(splits), _ptr(workspace), int(workspace_bytes), _ptr(A), _ptr(B),
                               _ptr(C), _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "gemm_splitk_run")


def gemm_splitk_run_noalloc(p: GemmPlan, splits: int, A, B, C, stream=None) -> None:
    """gemm_splitk_run_noalloc(): split-K through the library's fixed per-device scratch
    array (no workspace, no allocation); calls that overlap on one GPU race."""
    st = lib().gemm_splitk_run_noalloc(ctypes.byref(p), int(splits), _ptr(A), _ptr(B), _ptr(C),
                                       _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "gemm_splitk_run_noalloc")


def gemm_splitk(A, B, *, trans_a: bool = False, trans_b: bool = False, out_dtype=None, out=None,
                splits: Optional[int] = None, workspace=None, stream=None):
    """C = op(A) @ op(B) with K split into parts (gemm_splitk_run); splits defaults to
    tg_splitk_choose's suggestion.  The fp32 workspace is a caller tensor (allocated here
    when not given).  Returns C."""
    import torch
    _check_matrix(A, "A")
    _check_matrix(B, "B")
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    m, k = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    kb, n = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
    if kb != k:
        raise ValueError(f"inner dimensions differ: {k} vs {kb}")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=A.device)
    else:
        _check_out(out, (m, n), out_dtype)
    p = plan(m, n, k, trans_a=trans_a, trans_b=trans_b, in_dtype=A.dtype, out_dtype=out_dtype, lda=_ld(A),
             ldb=_ld(B), ldc=_ld(out))
    splits = splitk_choose(p) if splits is None else int(splits)
    need = splitk_workspace_bytes(p, splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=torch.float32, device=A.device)
    gemm_splitk_run(p, splits, workspace, workspace.numel() * workspace.element_size(), A, B, out, stream)
    return out


def bmm(A, B, *, trans_a: bool = False, trans_b: bool = False, out_dtype=None, out=None, stream=None):
    """C[b] = op(A[b]) @ op(B[b]) for 3-D tensors [batch, rows, cols] (batch stride from the tensor)."""
    import torch
    _check_matrix(A, "A", (3,))
    _check_matrix(B, "B", (3,))
    if A.shape[0] != B.shape[0]:
        raise ValueError("A and B must have the same batch")
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    batch = A.shape[0]
    m, k = (A.shape[2], A.shape[1]) if trans_a else (A.shape[1], A.shape[2])
    kb, n = (B.shape[2], B.shape[1]) if trans_b else (B.shape[1], B.shape[2])
    if kb != k:
        raise ValueError(f"inner dimensions differ: {k} vs {kb}")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((batch, m, n), dtype=out_dtype, device=A.device)
    else:
        _check_out(out, (batch, m, n), out_dtype, (3,))
    p = plan(m, n, k, trans_a=trans_a, trans_b=trans_b, in_dtype=A.dtype, out_dtype=out_dtype, lda=_ld(A),
             ldb=_ld(B), ldc=_ld(out), batch=max(batch, 1))
    bmm_run(p, batch, A.stride(0), B.stride(0), out.stride(0), A, B, out, stream)
    return out


def attention_fwd(in_type: int, out_type: int, batch: int, n_q: int, n_k: int, head_dim: int, scale: float,
                  Q, ldq: int, stride_q: int, K, ldk: int, stride_k: int, V, ldv: int, stride_v: int,
                  O, ldo: int, stride_o: int, stream=None) -> None:
    """attention_fwd(): raw call (dtype codes, pointers or tensors, element strides)."""
    st = lib().attention_fwd(in_type, out_type, batch, n_q, n_k, head_dim, ctypes.c_float(scale), _ptr(Q), ldq,
                             stride_q, _ptr(K), ldk, stride_k, _ptr(V), ldv, stride_v, _ptr(O), ldo, stride_o,
                             _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "attention_fwd")


def attention(Q, K, V, *, scale: Optional[float] = None, out_dtype=None, out=None, stream=None):
    """O = softmax(scale * Q K^T) V per head for 3-D tensors [batch, rows, head_dim]
    (head_dim contiguous); scale defaults to 1/sqrt(head_dim).  Returns O (new, or ``out``)."""
    import math
    import torch
    for X, name in ((Q, "Q"), (K, "K"), (V, "V")):
        _check_matrix(X, name, (3,))
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K and V must have the same dtype")
    batch, n_q, d = Q.shape
    if K.shape[0] != batch or V.shape[0] != batch or K.shape[2] != d or V.shape[2] != d or K.shape[1] != V.shape[1]:
        raise ValueError("K and V must be [batch, n_k, head_dim] with Q's batch and head_dim")
    n_k = K.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((batch, n_q, d), dtype=out_dtype, device=Q.device)
    else:
        _check_out(out, (batch, n_q, d), out_dtype, (3,))
    attention_fwd(_dtype_code(Q.dtype), _dtype_code(out_dtype), batch, n_q, n_k, d, scale, Q, _ld(Q), Q.stride(0),
                  K, _ld(K), K.stride(0), V, _ld(V), V.stride(0), out, _ld(out), out.stride(0), stream)
    return out


def group_tiles() -> int:
    """Tile shapes a grouped launch can be forced to (valid `tile` values of gemm_group_run)."""
    return int(lib().tg_group_tiles())


def gemm_group_run(in_type: int, out_type: int, trans_a: bool, trans_b: bool, problems, tile: int = -1,
                   stream=None) -> None:
    """gemm_group_run(): `problems` is a sequence of GroupProblem (or of 9-tuples
    m, n, k, lda, ldb, ldc, A, B, C with tensors or raw pointers)."""
    arr = (GroupProblem * max(len(problems), 1))()
    for i, q in enumerate(problems):
        if isinstance(q, GroupProblem):
            arr[i] = q
        else:
            m, n, k, lda, ldb, ldc, A, B, C = q
            arr[i] = GroupProblem(m, n, k, lda, ldb, ldc, _ptr(A) if A is not None else None,
                                  _ptr(B) if B is not None else None, _ptr(C) if C is not None else None)
    st = lib().gemm_group_run(in_type, out_type, int(trans_a), int(trans_b), arr, len(problems), tile,
                              _stream_handle(stream))
    if st != TG_OK:
        raise TgError(st, "gemm_group_run")


def gemm_group(As, Bs, *, trans_a: bool = False, trans_b: bool = False, out_dtype=None, outs=None, tile: int = -1,
               stream=None):
    """[op(A_i) @ op(B_i)] for lists of 2-D tensors of one dtype, in grouped launches; returns the outputs."""
    import torch
    if len(As) != len(Bs):
        raise ValueError("As and Bs differ in length")
    out_dtype = out_dtype or torch.float32
    probs, res = [], []
    for i, (A, B) in enumerate(zip(As, Bs)):
        _check_matrix(A, "A")
        _check_matrix(B, "B")
        if A.dtype != As[0].dtype or B.dtype != As[0].dtype:
            raise TypeError("all operands must have the same dtype")
        m, k = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
        kb, n = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
        if kb != k:
            raise ValueError(f"problem {i}: inner dimensions differ: {k} vs {kb}")
        if outs is not None:
            C = outs[i]
            _check_out(C, (m, n), out_dtype)
        else:
            C = torch.empty((m, n), dtype=out_dtype, device=A.device)
        probs.append((m, n, k, _ld(A), _ld(B), _ld(C), A, B, C))
        res.append(C)
    if probs:
        gemm_group_run(_dtype_code(As[0].dtype), _dtype_code(out_dtype), trans_a, trans_b, probs, tile, stream)
    return res
