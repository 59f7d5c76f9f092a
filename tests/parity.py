"""Acceptance rules for comparing the HIP path with the oracle, and GPU I/O helpers.

Tolerance for an fp32 result (per element):
    T = 2^-18 * K * max|a| * max|b|
with the maxima over the whole decoded A and B (every batch).  For a 16-bit
result the rounding of the fp32 sum adds at most half an output ulp:
    |C - Cref| <= T + ulp_out(|Cref| + T) / 2.
Integer-valued inputs whose partial sums stay below 2^24 are summed exactly
in fp32, so there the result must equal the oracle bit for bit (fp32) or the
nearest-even rounding of the exact sum (16-bit outputs).
"""
from __future__ import annotations

import numpy as np

import oracle

BF16_P, FP16_P = 8, 11          # significand bits incl. the hidden one
BF16_EMIN, FP16_EMIN = -126, -14


def tol_fp32(k: int, max_a: float, max_b: float) -> float:
    return 2.0 ** -18 * k * max_a * max_b


def half_ulp(x: np.ndarray, out_dtype: str) -> np.ndarray:
    p, emin = (BF16_P, BF16_EMIN) if out_dtype == "bf16" else (FP16_P, FP16_EMIN)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    return 0.5 * 2.0 ** (e - (p - 1))


def bound(cref: np.ndarray, t: float, out_dtype: str) -> np.ndarray:
    if out_dtype == "fp32":
        return np.full(cref.shape, t)
    return t + half_ulp(np.abs(cref) + t, out_dtype)


def check(c: np.ndarray, cref: np.ndarray, t: float, out_dtype: str, what: str = "") -> float:
    """Assert the rule; return the worst |C - Cref| / bound for reporting."""
    assert c.shape == cref.shape, (c.shape, cref.shape)
    assert np.all(np.isfinite(c)), f"{what}: non-finite output"
    b = bound(cref, t, out_dtype)
    err = np.abs(c - cref)
    bad = err > b
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements over tolerance, e.g. at {idx.tolist()}: "
                             f"got {c[bad][:5]}, want {cref[bad][:5]}, bound {b[bad][:5]}")
    return float(np.max(err / np.maximum(b, 1e-300))) if err.size else 0.0


def check_exact(c_bits_or_vals: np.ndarray, cref: np.ndarray, out_dtype: str, what: str = "") -> None:
    if out_dtype == "fp32":
        assert np.array_equal(c_bits_or_vals.astype(np.float64), cref), f"{what}: not bit-exact"
    else:
        want = oracle.round_to(cref, out_dtype)
        assert np.array_equal(c_bits_or_vals, want), f"{what}: not the nearest-even rounding of the exact sum"


# ------------------------------------------------------------ GPU I/O ---

def to_gpu(bits: np.ndarray, in_dtype: str = "bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if in_dtype == "bf16" else torch.float16).cuda()


def torch_out_dtype(out_dtype: str):
    import torch
    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[out_dtype]


def values(c) -> np.ndarray:
    """GPU result -> float64 numpy (exact widening)."""
    import torch
    return c.detach().to(torch.float64).cpu().numpy()


def bits(c) -> np.ndarray:
    import torch
    return c.detach().cpu().view(torch.int16).numpy().view(np.uint16)
