"""The epilogue's fp32 -> bf16 / fp16 rounding, bit for bit, in every kernel
that writes a 16-bit C.

Each output is made to hold a chosen fp32 value t exactly before rounding:
t is split into three 16-bit pieces h + m + l (h the leading bits of t, m the
next, l the rest, each exactly representable in the input type), A carries
the pieces of output j of row i in columns 3j, 3j+1, 3j+2, and B is the
0/1 matrix with B[3j + r][j] = 1.  Every product is exact and every partial
sum is a shorter piece of t, so the fp32 accumulator holds t whatever the
order of additions, and the stored 16-bit value must be the nearest-even
rounding of t (the reading of the unstated rounding mode; the oracle's
encoder is pinned against torch and numpy on the CPU).  The targets cover
every pattern of the bits that rounding drops, with both parities of the
last kept bit (exact ties round to even), both signs, several exponents,
and values that round up to infinity.
"""
import ctypes

import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
from parity import bits, to_gpu, torch_out_dtype

pytestmark = pytest.mark.gpu

KEEP = {"bf16": 8, "fp16": 11}   # significand bits of the 16-bit type (hidden bit included)


def _trunc(x: np.ndarray, keep: int) -> np.ndarray:
    """x cut toward zero to `keep` significant bits (float64, exact)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    q = 2.0 ** (e - (keep - 1))
    return np.where(ax > 0, np.sign(x) * np.floor(ax / q) * q, 0.0)


def targets(dtype: str, count: int) -> np.ndarray:
    """`count` fp32 values (as float64) whose dropped low bits run through
    every pattern, each with both parities of the last kept bit; past the
    first 2^(dropped bits + 1) values, exact ties and their two neighbours."""
    drop = 24 - KEEP[dtype]                          # fp32 significand bits lost by the rounding
    low = np.arange(count, dtype=np.uint64) % (1 << drop)
    extra = np.arange(count) >= (2 << drop)
    half = np.uint64(1 << (drop - 1))
    low[extra] = half + (np.arange(count, dtype=np.int64)[extra] % 3 - 1).astype(np.uint64)
    par = (np.arange(count, dtype=np.uint64) >> drop) & 1
    par[extra] = np.random.default_rng(98).integers(0, 2, int(extra.sum())).astype(np.uint64)
    rng = np.random.default_rng(99)
    mid = rng.integers(0, 1 << (KEEP[dtype] - 2), count).astype(np.uint64)   # other kept bits
    # exponents: mostly moderate, some near the top of the range so that a
    # round-up reaches infinity (kept bits all ones)
    if dtype == "bf16":
        exps = rng.integers(100, 160, count).astype(np.uint64)
        top = np.arange(count) % 64 == 5
        exps[top] = 254
    else:
        exps = rng.integers(126, 141, count).astype(np.uint64)              # |t| in [2^-1, 2^14): pieces exact
        top = np.arange(count) % 64 == 5
        exps[top] = 142                                                       # [2^15, 2^16): fp16 max 65504
    mid[top] = (1 << (KEEP[dtype] - 2)) - 1
    par[top] = 1
    sign = (np.arange(count, dtype=np.uint64) >> (drop + 1)) & 1
    frac = (mid << np.uint64(drop + 1)) | (par << np.uint64(drop)) | low     # 23 fraction bits
    u = (sign << np.uint64(31)) | (exps << np.uint64(23)) | frac
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def pieces(t: np.ndarray, dtype: str) -> np.ndarray:
    """[count, 3] 16-bit patterns of h, m, l with h + m + l == t exactly."""
    keep = KEEP[dtype]
    h = _trunc(t, keep)
    m = _trunc(t - h, keep)
    l = t - h - m
    out = np.stack([h, m, l], 1)
    tt = torch.from_numpy(out)
    enc = tt.to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    assert torch.equal(enc.double(), tt), "a piece is not exact in the input type"
    assert np.array_equal(h + m + l, t)
    return enc.view(torch.int16).numpy().view(np.uint16)


def operands(dtype: str, rows: int, per_row: int, trans_b: bool):
    t = targets(dtype, rows * per_row)
    P = pieces(t, dtype).reshape(rows, 3 * per_row)                   # A: rows x 3*per_row
    one = np.uint16(0x3F80) if dtype == "bf16" else np.uint16(0x3C00)
    sel = np.zeros((3 * per_row, per_row), np.uint16)                 # B[3j + r][j] = 1
    for r in range(3):
        sel[np.arange(per_row) * 3 + r, np.arange(per_row)] = one
    B = np.ascontiguousarray(sel.T) if trans_b else sel
    return P, B, t.reshape(rows, per_row)


def run(dtype, rows, per_row, trans_b=False, variant=None, tile=None, splits=None):
    A, B, t = operands(dtype, rows, per_row, trans_b)
    m, n, k = rows, per_row, 3 * per_row
    tin = torch.bfloat16 if dtype == "bf16" else torch.float16
    C = torch.empty((m, n), dtype=torch_out_dtype(dtype), device="cuda")
    p = tg.plan(m, n, k, trans_b=trans_b, in_dtype=tin, out_dtype=tin)
    if variant is not None:
        p = tg.plan_tile(p, variant, tile)
    Ag, Bg = to_gpu(A, dtype), to_gpu(B, dtype)
    print(f"rounding case {dtype} m={m} n={n} k={k} tb={trans_b} variant={p.variant} tile={p.tile} "
          f"splits={splits}", flush=True)
    if splits:
        need = tg.splitk_workspace_bytes(p, splits)
        ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device="cuda")
        tg.gemm_splitk_run(p, splits, ws, need, Ag, Bg, C)
    else:
        tg.gemm_run(p, Ag, Bg, C)
    torch.cuda.synchronize()
    cref = oracle.gemm(A, B, m=m, n=n, k=k, trans_b=int(trans_b), in_dtype=dtype)[0]
    assert np.array_equal(cref, t), "the oracle's product is not the chosen target"
    want = oracle.round_to(cref, dtype)
    got = bits(C)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{bad.shape[0]} roundings differ, e.g. t = {t[tuple(bad[0])]!r}: "
                           f"got 0x{int(got[tuple(bad[0])]):04x}, want 0x{int(want[tuple(bad[0])]):04x}")
    return p


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_tile_kernels(dtype):
    # 544 x 256 outputs: 2 x 65536 targets (bf16 drops 16 bits: every pattern, both parities),
    # then 8192 ties and neighbours of ties
    p = run(dtype, 544, 256)
    assert p.variant == tg.VARIANT_TILE
    for tile in (0, 1, 4, 11, tg.TILE_KSLICE):
        run(dtype, 544, 256, variant=tg.VARIANT_TILE, tile=tile)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_pingpong_kernel(dtype):
    run(dtype, 544, 256, variant=tg.VARIANT_TILE, tile=tg.TILE_PINGPONG)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_skinny_kernel(dtype):
    # 32 rows x 4352 outputs, B stored N x K (both operands K-contiguous)
    p = run(dtype, 32, 4352, trans_b=True)
    assert p.variant == tg.VARIANT_SKINNY
    run(dtype, 16, 8704, trans_b=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_panel_kernel(dtype):
    # K = 3 x 40 = 120 <= 128: the panel kernel's range
    run(dtype, 3480, 40, variant=tg.VARIANT_TILE, tile=tg.TILE_PANEL)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_element_wise_kernel_and_splitk_reduction(dtype):
    run(dtype, 544, 256, variant=tg.VARIANT_GENERIC, tile=0)
    run(dtype, 544, 256, splits=3)
