"""The panel kernel (TG_TILE_PANEL, short K) against the oracle.

It is forced onto shapes that exercise every path of it:
- M tails: rows past M in a 128-row panel read as zero and are never stored.
- N tails inside a 128-column tile.
- K = 8 .. 128: slices past K are skipped, and K-contiguous units past K are zero-filled.
- Both B layouts (stored K x N, and N x K).
- bf16 and fp16 inputs; fp32 and 16-bit outputs (two staged row bands, and one).
- Batches with padded ldc.
- Runs split over a row panel, including a last run shorter than the rest.
- Integer inputs, which must match bit for bit.
- Batches that share an operand through a zero batch stride, for the panel
  kernel and for the tile kernel's non-temporal loads of unshared operands.
- Every case the launcher hands to the 128 x 128 tile kernel instead: an
  epilogue, A stored K x M, K > 128, K = 0, and N not a whole number of
  16-byte output units.
"""
import ctypes

import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
import synth
from parity import bits, check, check_exact, to_gpu, tol_fp32, torch_out_dtype, values

pytestmark = pytest.mark.gpu

CANARY = -12345.0


def run(m, n, k, ta, tb, out_dtype, batch=1, seed=0, dist=("normal", 1.0), in_dtype="bf16", ldc_pad=0, idx=None):
    """Forced panel-tile run; returns (C values [batch, m, n], oracle values at idx or full, A, B, C buffer)."""
    rng = np.random.default_rng(seed)
    ar, ac = (k, m) if ta else (m, k)
    br, bc = (n, k) if tb else (k, n)
    A = synth.draw(rng, (batch, ar, ac), *dist, dtype=in_dtype)
    B = synth.draw(rng, (batch, br, bc), *dist, dtype=in_dtype)
    tin = torch.bfloat16 if in_dtype == "bf16" else torch.float16
    tout = torch_out_dtype(out_dtype)
    ldc = n + ldc_pad
    Cbuf = torch.full((batch, m, ldc), CANARY, dtype=tout, device="cuda")
    pl = tg.plan(m, n, k, trans_a=ta, trans_b=tb, in_dtype=tin, out_dtype=tout, ldc=ldc, batch=batch)
    pl = tg.plan_tile(pl, tg.VARIANT_TILE, tg.TILE_PANEL)
    Ag, Bg = to_gpu(A, in_dtype), to_gpu(B, in_dtype)
    st = tg.lib().bmm_run(ctypes.byref(pl), batch, ar * ac, br * bc, m * ldc, Ag.data_ptr(), Bg.data_ptr(),
                          Cbuf.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.status_str(st)
    torch.cuda.synchronize()
    cb = values(Cbuf)
    canary = float(torch.tensor(CANARY, dtype=tout).item())
    assert np.all(cb[:, :, n:] == canary), "wrote into the ldc padding"
    ref = oracle.gemm(A, B, m=m, n=n, k=k, trans_a=ta, trans_b=tb, batch=batch, stride_a=ar * ac,
                      stride_b=br * bc, in_dtype=in_dtype, idx=idx)
    return cb[:, :, :n], ref, A, B, Cbuf


SHAPES = [(296, 520, 128), (128, 512, 64), (200, 264, 8), (136, 1032, 120), (384, 384, 16), (8, 16, 40)]


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("tb", [0, 1])
def test_tails_both_b_layouts(tb, out_dtype):
    for i, (m, n, k) in enumerate(SHAPES):
        got, ref, A, B, _ = run(m, n, k, 0, tb, out_dtype, seed=i, ldc_pad=8 * (i % 2))
        check(got[0], ref[0], tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), out_dtype,
              f"panel m={m} n={n} k={k} tb={tb} {out_dtype}")


@pytest.mark.parametrize("tb", [0, 1])
def test_integer_inputs_bit_exact(tb):
    for out_dtype in ("fp32", "bf16"):
        got, ref, *_, Cbuf = run(264, 1032, 128, 0, tb, out_dtype, batch=2, seed=3, dist=("int", -8, 8))
        if out_dtype == "fp32":
            check_exact(got, ref, "fp32", "panel int")
        else:
            check_exact(bits(Cbuf).reshape(2, 264, 1032), ref, "bf16", "panel int bf16")


@pytest.mark.parametrize("out_dtype", ["fp32", "fp16"])
def test_fp16_inputs(out_dtype):
    for tb in (0, 1):
        got, ref, A, B, _ = run(264, 640, 96, 0, tb, out_dtype, seed=5, in_dtype="fp16")
        check(got[0], ref[0], tol_fp32(96, oracle.max_abs(A, "fp16"), oracle.max_abs(B, "fp16")), out_dtype,
              f"panel fp16 tb={tb}")


def test_runs_split_over_a_panel():
    """One 128-row panel of 40 column tiles: the launcher splits it into runs
    of 3 tiles (the last one a single tile) to give the CUs more work-groups."""
    got, ref, A, B, _ = run(128, 40 * 128, 64, 0, 1, "fp32", seed=11, dist=("int", -4, 4))
    check_exact(got, ref, "fp32", "panel runs")


def test_batches_sampled():
    """A batch of 96 score-like products (K = 128, B stored N x K), sampled."""
    m, n, k, batch = 512, 512, 128, 96
    idx = synth.sample_indices(12, batch, m, n, count=4096)
    got, ref, A, B, _ = run(m, n, k, 0, 1, "fp32", batch=batch, seed=12, idx=idx)
    check(got[idx[:, 0], idx[:, 1], idx[:, 2]], ref, tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), "fp32",
          "panel batch=96")


@pytest.mark.parametrize("case", ["trans_a", "k_200", "k_0", "n_odd"])
def test_cases_handed_to_the_tile_kernel(case):
    m, n, k, ta, tb, pad = {"trans_a": (264, 264, 128, 1, 0, 0), "k_200": (264, 264, 200, 0, 1, 0),
                            "k_0": (264, 264, 0, 1, 0, 0), "n_odd": (264, 263, 64, 0, 1, 1)}[case]
    got, ref, A, B, _ = run(m, n, k, ta, tb, "fp32", seed=13, ldc_pad=pad)
    if k == 0:
        assert np.all(got == 0.0)
        return
    check(got[0], ref[0], tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), "fp32", f"panel fallback {case}")


def test_epilogue_goes_to_the_tile_kernel():
    rng = np.random.default_rng(21)
    m, n, k = 264, 520, 64
    A = synth.draw(rng, (1, m, k), "int", -3, 3)
    B = synth.draw(rng, (1, k, n), "int", -3, 3)
    C0 = rng.integers(-8, 9, size=(1, m, n)).astype(np.float32)
    Cg = torch.from_numpy(C0.copy()).cuda()
    pl = tg.plan(m, n, k, out_dtype=torch.float32)
    pl = tg.plan_tile(pl, tg.VARIANT_TILE, tg.TILE_PANEL)
    tg.bmm_run_ex(pl, 1, m * k, k * n, m * n, to_gpu(A), to_gpu(B), Cg, alpha=2.0, beta=-1.0)
    torch.cuda.synchronize()
    P = oracle.gemm(A, B, m=m, n=n, k=k)
    check_exact(values(Cg), oracle.epilogue(P, 2.0, -1.0, C0.astype(np.float64), None), "fp32", "panel epilogue")


@pytest.mark.parametrize("case", ["panel_shared_B", "one_column_shared_A", "one_column_own_A"])
def test_batches_that_share_an_operand(case):
    """A zero batch stride shares one operand between the batch's products.
    The panel kernel reads it per run. With one column of tiles, the launcher
    loads A non-temporally only when no other matrix of the batch reads it."""
    rng = np.random.default_rng(41)
    batch = 3
    if case == "panel_shared_B":
        m, n, k, tb, tile = 264, 640, 128, 1, tg.TILE_PANEL
        A = synth.draw(rng, (batch, m, k), "int", -4, 4)
        B = synth.draw(rng, (n, k), "int", -4, 4)
        sA, sB = m * k, 0
    else:
        m, n, k, tb, tile = 520, 128, 1000, 0, 4  # the 128 x 128 tile kernel
        A = synth.draw(rng, (m, k) if case == "one_column_shared_A" else (batch, m, k), "int", -4, 4)
        B = synth.draw(rng, (batch, k, n), "int", -4, 4)
        sA, sB = (0 if case == "one_column_shared_A" else m * k), k * n
    pl = tg.plan_tile(tg.plan(m, n, k, trans_b=tb, batch=batch), tg.VARIANT_TILE, tile)
    C = torch.empty((batch, m, n), dtype=torch.float32, device="cuda")
    tg.bmm_run(pl, batch, sA, sB, m * n, to_gpu(A), to_gpu(B), C)
    torch.cuda.synchronize()
    ref = oracle.gemm(A, B, m=m, n=n, k=k, trans_b=tb, batch=batch, stride_a=sA, stride_b=sB)
    check_exact(values(C), ref, "fp32", case)
