"""The alpha/beta/bias epilogue (gemm_run_ex, bmm_run_ex) against the oracle.

Tolerance: the kernel forms alpha*acc, then fma(beta, C, .), then + bias, in
fp32, from an accumulator within T = 2^-18 K max|a| max|b| of the exact
product (parity.py); so
    |C - Cref| <= |alpha| T + 3 * 2^-24 (|alpha P| + |beta C| + |bias|)
plus half an output ulp for 16-bit outputs.  Integer-valued data keep every
step exact, so there the result must match the oracle bit for bit (or its
nearest-even rounding).  Covered: the tile, element-wise and skinny kernels,
batches (one bias for all), K = 0, beta = 0 with NaN in C (C is not read),
bias alone, and plans whose persistent flags the epilogue switches off.
"""
import ctypes

import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
import synth
from parity import bound, check_exact, to_gpu, tol_fp32, torch_out_dtype, values

pytestmark = pytest.mark.gpu


def dec(bits, dtype):
    return oracle.decode(bits, dtype) if dtype != "fp32" else bits


def run(m, n, k, ta, tb, out_dtype, alpha, beta, use_bias, seed, dist=("normal", 1.0), batch=1, pad_a=0,
        nan_c=False, exact=False, clear_flags=0):
    rng = np.random.default_rng(seed)
    ar, ac = (k, m) if ta else (m, k)
    br, bc = (n, k) if tb else (k, n)
    lda, ldb, ldc = max(ac, 1) + pad_a, max(bc, 1), max(n, 1)
    A = np.zeros((batch, ar, lda), dtype=np.uint16)
    A[:, :, :ac] = synth.draw(rng, (batch, ar, ac), *dist)
    B = synth.draw(rng, (batch, br, bc), *dist)
    tout = torch_out_dtype(out_dtype)
    if out_dtype == "fp32":
        C0 = (rng.integers(-8, 9, size=(batch, m, n)).astype(np.float32) if exact
              else rng.standard_normal((batch, m, n)).astype(np.float32))
        C0v = C0.astype(np.float64)
        Cg = torch.from_numpy(C0.copy()).cuda()
    else:
        c_bits = synth.draw(rng, (batch, m, n), *(("int", -8, 8) if exact else ("normal", 1.0)), dtype=out_dtype)
        C0v = oracle.decode(c_bits, out_dtype)
        Cg = to_gpu(c_bits, out_dtype)
    if nan_c:
        Cg.fill_(float("nan"))
    bias_v = None
    bias_g = None
    if use_bias:
        if out_dtype == "fp32":
            bv = rng.integers(-4, 5, size=n).astype(np.float32) if exact else rng.standard_normal(n).astype(np.float32)
            bias_v = bv.astype(np.float64)
            bias_g = torch.from_numpy(bv).cuda()
        else:
            bb = synth.draw(rng, (n,), *(("int", -4, 4) if exact else ("normal", 1.0)), dtype=out_dtype)
            bias_v = oracle.decode(bb, out_dtype)
            bias_g = to_gpu(bb, out_dtype)
    Ag, Bg = to_gpu(A), to_gpu(B)
    pl = tg.plan(m, n, k, trans_a=ta, trans_b=tb, out_dtype=tout, lda=lda, ldb=ldb, ldc=ldc, batch=batch)
    pl.flags &= ~clear_flags
    if batch == 1:
        tg.gemm_run_ex(pl, Ag, Bg, Cg, alpha=alpha, beta=beta, bias=bias_g)
    else:
        tg.bmm_run_ex(pl, batch, ar * lda, br * bc, m * n, Ag, Bg, Cg, alpha=alpha, beta=beta, bias=bias_g)
    torch.cuda.synchronize()
    P = oracle.gemm(A, B, m=m, n=n, k=k, trans_a=ta, trans_b=tb, lda=lda, ldb=bc, batch=batch,
                    stride_a=ar * lda, stride_b=br * bc)
    ref = oracle.epilogue(P, alpha, beta, C0v, bias_v)
    what = f"{m}x{n}x{k} ta={ta} tb={tb} {out_dtype} a={alpha} b={beta} bias={use_bias} variant={pl.variant}"
    if exact:
        if out_dtype == "fp32":
            check_exact(values(Cg), ref, out_dtype, what)
        else:
            check_exact(Cg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), ref, out_dtype, what)
        return pl
    got = values(Cg)
    assert np.all(np.isfinite(got)), what
    t = abs(alpha) * (tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)) if k else 0.0)
    mag = np.abs(alpha * P) + (np.abs(beta * C0v) if beta != 0 else 0) + (np.abs(bias_v) if use_bias else 0)
    t = t + 3 * 2.0 ** -24 * mag
    b = bound(ref, t, out_dtype)
    err = np.abs(got - ref)
    assert np.all(err <= b), f"{what}: worst {float(np.max(err / b)):.3g}x the bound"
    return pl


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_epilogue_tile_kernel(ta, tb, out_dtype):
    pl = run(200, 264, 136, ta, tb, out_dtype, 0.75, -1.25, True, seed=ta * 2 + tb)
    assert pl.variant == tg.VARIANT_TILE


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_epilogue_generic_kernel(out_dtype):
    pl = run(67, 45, 33, 0, 0, out_dtype, -2.0, 0.5, True, seed=11, pad_a=3)
    assert pl.variant == tg.VARIANT_GENERIC


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_epilogue_skinny_kernel(out_dtype):
    pl = run(16, 1000, 512, 0, 1, out_dtype, 1.5, 2.0, True, seed=12)
    assert pl.variant == tg.VARIANT_SKINNY


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_epilogue_integer_data_bit_exact(out_dtype):
    for (m, n, k, ta, tb) in [(128, 256, 64, 0, 0), (16, 512, 256, 0, 1), (37, 41, 29, 1, 0)]:
        run(m, n, k, ta, tb, out_dtype, 2.0, -1.0, True, seed=m + n, dist=("int", -3, 3), exact=True)


def test_epilogue_beta_zero_ignores_nan_in_c():
    run(128, 128, 64, 0, 0, "fp32", 3.0, 0.0, True, seed=13, nan_c=True)
    run(16, 256, 128, 0, 1, "bf16", 3.0, 0.0, False, seed=14, nan_c=True)


def test_epilogue_k0_gives_beta_c_plus_bias():
    run(64, 72, 0, 0, 0, "fp32", 5.0, 0.25, True, seed=15)


def test_epilogue_batched_bias_broadcast():
    run(96, 136, 72, 0, 1, "bf16", 0.5, 1.0, True, seed=16, batch=3)


def test_epilogue_bias_only_and_persistent_flags_ignored():
    """A large plan with persistent launch flags: the epilogue runs without
    them, and the result equals the run with them cleared."""
    flags = tg.FLAG_PERSIST | tg.FLAG_PREFETCH
    pl = run(2048, 2048, 256, 0, 0, "fp32", 1.0, 0.0, True, seed=17, dist=("int", -2, 2), exact=True)
    assert pl.flags & tg.FLAG_PERSIST
    run(2048, 2048, 256, 0, 0, "fp32", 1.0, 0.0, True, seed=17, dist=("int", -2, 2), exact=True, clear_flags=flags)


def test_epilogue_misaligned_bias_rejected():
    pl = tg.plan(64, 64, 64)
    A = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    bias = torch.zeros(65, dtype=torch.float32, device="cuda")
    e = tg.Epilogue(1.0, 0.0, bias.data_ptr() + 2)
    st = tg.lib().gemm_run_ex(ctypes.byref(pl), ctypes.byref(e), A.data_ptr(), A.data_ptr(), C.data_ptr(), None)
    assert st == tg.TG_ERR_INVALID


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_epilogue_on_a_256x128_plan(out_dtype):
    """An O = P V shaped batch (HBM-bound, N = 128, 256 work items) is planned
    onto the 256 x 128 entry; with an epilogue the launcher sends it to the
    128 x 128 epilogue twin.  Integer data: bit for bit."""
    pl = run(512, 128, 128, 0, 0, out_dtype, 2.0, -1.0, True, seed=18, dist=("int", -3, 3), batch=128, exact=True)
    assert (pl.variant, pl.tile, pl.bm, pl.bn) == (tg.VARIANT_TILE, 17, 256, 128)
