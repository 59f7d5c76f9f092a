"""Algorithmic work, traffic and roofline figures for a GEMM/BMM call.

Counting follows "Optimize Triton Block Parameters" (Step 1): 2*M*N*K flops
per matrix, and the bytes of reading A and B once and writing C once; the
arithmetic intensity flops/bytes placed against the ridge point
peak_flops / peak_bandwidth decides whether the call is bound by the matrix
cores or by HBM.  Step 2 of the same page gives the on-chip staging budget as
the A and B tiles times the number of pipeline stages.
"""
from __future__ import annotations

# MI355X (gfx950) published peaks: 256 CUs at 2.4 GHz.
MI355X_BF16_DENSE_FLOPS = 2.5e15   # dense bf16/fp16 MFMA, FLOP/s
MI355X_HBM_BYTES = 8.0e12          # HBM3E, B/s
MI355X_LDS_PER_WORKGROUP = 160 * 1024


def gemm_flops(m: int, n: int, k: int, batch: int = 1) -> int:
    return 2 * m * n * k * batch


def gemm_bytes(m: int, n: int, k: int, in_size: int = 2, out_size: int = 4, batch: int = 1) -> int:
    """Read A (M x K) and B (K x N) once, write C (M x N) once."""
    return batch * ((m * k + k * n) * in_size + m * n * out_size)


def intensity(m, n, k, in_size=2, out_size=4, batch=1) -> float:
    return gemm_flops(m, n, k, batch) / gemm_bytes(m, n, k, in_size, out_size, batch)


def ridge(peak_flops: float, peak_bytes: float) -> float:
    return peak_flops / peak_bytes


def bound(m, n, k, in_size=2, out_size=4, batch=1, peak_flops=MI355X_BF16_DENSE_FLOPS,
          peak_bytes=MI355X_HBM_BYTES) -> str:
    return "mfma" if intensity(m, n, k, in_size, out_size, batch) >= ridge(peak_flops, peak_bytes) else "hbm"


def lds_budget(bm: int, bn: int, bk: int, stages: int, elem: int = 2) -> int:
    """Bytes of on-chip staging: stages x (A tile + B tile)."""
    return stages * (bm * bk + bk * bn) * elem


def accumulator_bytes(bm: int, bn: int, acc_size: int = 4) -> int:
    return bm * bn * acc_size
