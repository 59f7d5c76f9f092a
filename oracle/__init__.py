"""CPU oracle for the tiled GEMM/BMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library under test never does, and this
package imports nothing from it.

The arithmetic lives in ``oracle_gemm.c`` (plain C, fp64 accumulation over
exactly decoded bf16/fp16 inputs, one sequential k-loop per output element);
this file only builds it with gcc and marshals numpy arrays through ctypes.

What it follows: C[b] = op(A[b]) op(B[b]) with op() a stride swap and the batch
a per-operand base offset (p1 "Triton Optimization Reference" sections 2 and 3;
p2 "Optimize Triton Block Parameters" Step 1 for the 2*M*N*K flop count); and,
for the fused attention forward pass, O = softmax(scale * Q K^T) V row by row
with no mask (``oracle_attention.c``; p1's opening section names attention as
the companion of its GEMM/BMM patterns).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_SRC_ATTN = os.path.join(_HERE, "oracle_attention.c")
_LIB = os.path.join(_HERE, "liboracle.so")

IN_TYPES = {"bf16": 0, "fp16": 1}
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (host only, no HIP)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_ATTN))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, _SRC_ATTN, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                    p, i64, i64, p, i64, i64, i64, p, i64, p]
        lib.oracle_max_abs.restype = ctypes.c_double
        lib.oracle_max_abs.argtypes = [ctypes.c_int, p, i64]
        lib.oracle_decode.restype = None
        lib.oracle_decode.argtypes = [ctypes.c_int, p, i64, p]
        lib.oracle_round.restype = None
        lib.oracle_round.argtypes = [ctypes.c_int, p, i64, p]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.c_double, p, i64, i64, p, i64, i64,
                                         p, i64, i64, i64, p, i64, p]
        _lib = lib
    return _lib


def _u16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {x.dtype}")
    return x


def _ptr(x: np.ndarray):
    return ctypes.c_void_p(x.ctypes.data) if x.size else ctypes.c_void_p(0)


def gemm(A: np.ndarray, B: np.ndarray, *, m: int, n: int, k: int, trans_a: int = 0, trans_b: int = 0,
         lda: int = 0, ldb: int = 0, batch: int = 1, stride_a: int = 0, stride_b: int = 0,
         in_dtype: str = "bf16", idx: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 reference.  Returns [batch, m, n] (full) or [len(idx)] (sampled).

    ``A`` and ``B`` are flat-addressable uint16 bit patterns; ``idx`` holds
    (b, i, j) rows.
    """
    lib = _load()
    A = _u16(A)
    B = _u16(B)
    lda = lda or (m if trans_a else k)
    ldb = ldb or (k if trans_b else n)
    if idx is None:
        out = np.empty((batch, m, n), dtype=np.float64)
        ip, ni = ctypes.c_void_p(0), 0
    else:
        idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 3)
        out = np.empty(idx.shape[0], dtype=np.float64)
        ip, ni = _ptr(idx), idx.shape[0]
    rc = lib.oracle_gemm(IN_TYPES[in_dtype], int(trans_a), int(trans_b), m, n, k, _ptr(A), lda,
                         stride_a, _ptr(B), ldb, stride_b, batch, ip, ni, _ptr(out))
    if rc != 0:
        raise IndexError("oracle_gemm: sample index outside the problem")
    return out


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, *, n_q: int, n_k: int, head_dim: int, scale: float,
              batch: int = 1, ldq: int = 0, ldk: int = 0, ldv: int = 0, sq: int = 0, sk: int = 0, sv: int = 0,
              in_dtype: str = "bf16", rows: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 reference of softmax(scale * Q K^T) V, no mask (oracle_attention.c).

    Q, K, V are flat-addressable uint16 bit patterns, row-major with head_dim
    contiguous.  Returns [len(rows), head_dim] for the requested (b, i) rows,
    or [batch, n_q, head_dim] when ``rows`` is None.
    """
    lib = _load()
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    ldq, ldk, ldv = ldq or head_dim, ldk or head_dim, ldv or head_dim
    sq, sk, sv = sq or n_q * ldq, sk or n_k * ldk, sv or n_k * ldv
    full = rows is None
    if full:
        bb, ii = np.meshgrid(np.arange(batch), np.arange(n_q), indexing="ij")
        rows = np.stack([bb.ravel(), ii.ravel()], 1)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    out = np.empty((rows.shape[0], head_dim), dtype=np.float64)
    rc = lib.oracle_attention(IN_TYPES[in_dtype], n_q, n_k, head_dim, float(scale), _ptr(Q), ldq, sq, _ptr(K), ldk,
                              sk, _ptr(V), ldv, sv, batch, _ptr(rows), rows.shape[0], _ptr(out))
    if rc != 0:
        raise IndexError("oracle_attention: row outside the problem, n_k < 1, or out of memory")
    return out.reshape(batch, n_q, head_dim) if full else out


def epilogue(P: np.ndarray, alpha: float = 1.0, beta: float = 0.0, C_in: Optional[np.ndarray] = None,
             bias: Optional[np.ndarray] = None) -> np.ndarray:
    """alpha * P + beta * C_in + bias[j], elementwise in fp64 (the scaled-and-shifted
    product the pages call a trivial epilogue: "Finetuning Your Program", the
    alpha/beta note).  P: the exact product from gemm() (any leading shape,
    columns last); C_in: prior contents of C as values (read only when
    beta != 0, as BLAS defines it: with beta = 0, NaN or Inf in C never
    reach the result); bias: one value per column, added to every row."""
    out = float(alpha) * np.asarray(P, dtype=np.float64)
    if beta != 0.0:
        out = out + float(beta) * np.asarray(C_in, dtype=np.float64)
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64).reshape((1,) * (out.ndim - 1) + (-1,))
    return out


def gemm_problem(p, idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Reference for a ``synth.Problem``."""
    return gemm(p.A, p.B, m=p.m, n=p.n, k=p.k, trans_a=p.trans_a, trans_b=p.trans_b, lda=p.lda,
                ldb=p.ldb, batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b,
                in_dtype=p.in_dtype, idx=idx)


def max_abs(X: np.ndarray, in_dtype: str = "bf16") -> float:
    X = _u16(X)
    return float(_load().oracle_max_abs(IN_TYPES[in_dtype], _ptr(X), X.size))


def decode(X: np.ndarray, in_dtype: str = "bf16") -> np.ndarray:
    X = _u16(X)
    out = np.empty(X.shape, dtype=np.float64)
    _load().oracle_decode(IN_TYPES[in_dtype], _ptr(X), X.size, _ptr(out))
    return out


def round_to(x: np.ndarray, out_dtype: str) -> np.ndarray:
    """Round doubles to bf16/fp16 bit patterns, nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_round(IN_TYPES[out_dtype], _ptr(x), x.size, _ptr(out))
    return out
