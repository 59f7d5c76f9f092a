"""The ping-pong kernel (TG_TILE_PINGPONG / TG_TILE_PINGPONG_EPI) against the oracle.

It is the planner's choice for large MFMA-bound products (the 8192^3 workload
is checked in test_parity.py); here it is forced onto shapes that exercise
every path of it: M/N tails inside a 256 x 256 tile, K tails inside a 64-deep
step (zero-filled K-contiguous units), K shorter than one step, all four
transposes, bf16 and fp16 inputs, fp32 and 16-bit outputs, batches, the
persistent launch (several tiles per work-group, the stores of one tile
issued during the next tile's first step) against one work-group per tile,
N not a multiple of 4 (no persistent launch, element-wise tail stores), the
epilogue entry, and K = 0 (handed to the 8-wave tile kernel).
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
PERSIST = tg.FLAG_PERSIST


def run(m, n, k, ta, tb, out_dtype, batch=1, seed=0, dist=("normal", 1.0), in_dtype="bf16", flags=None,
        ldc_pad=0, idx=None):
    """Forced ping-pong run; returns (C values [batch, m, n], oracle values at idx or full, A, B)."""
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
    pl = tg.plan_tile(pl, tg.VARIANT_TILE, tg.TILE_PINGPONG)
    if flags is not None:
        pl.flags = (pl.flags & ~PERSIST) | flags
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


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_tails_every_transpose(ta, tb, out_dtype):
    for i, (m, n, k) in enumerate([(296, 264, 200), (256, 256, 64), (520, 264, 1000), (8, 16, 8),
                                   (264, 520, 40), (512, 512, 136)]):
        got, ref, A, B, _ = run(m, n, k, ta, tb, out_dtype, seed=i, ldc_pad=8 * (i % 2))
        check(got[0], ref[0], tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), out_dtype,
              f"pingpong m={m} n={n} k={k} ta={ta} tb={tb} {out_dtype}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_integer_inputs_bit_exact(ta, tb):
    for out_dtype in ("fp32", "bf16"):
        got, ref, *_ , Cbuf = run(264, 296, 328, ta, tb, out_dtype, seed=3, dist=("int", -8, 8))
        if out_dtype == "fp32":
            check_exact(got[0], ref[0], "fp32", "pingpong int")
        else:
            raw = bits(Cbuf).reshape(1, 264, 296)
            check_exact(raw[0], ref[0], "bf16", "pingpong int bf16")


@pytest.mark.parametrize("out_dtype", ["fp32", "fp16"])
def test_fp16_inputs(out_dtype):
    for ta, tb in [(0, 0), (1, 1)]:
        got, ref, A, B, _ = run(264, 264, 200, ta, tb, out_dtype, seed=5, in_dtype="fp16")
        check(got[0], ref[0], tol_fp32(200, oracle.max_abs(A, "fp16"), oracle.max_abs(B, "fp16")), out_dtype,
              f"pingpong fp16 ta={ta} tb={tb}")


@pytest.mark.parametrize("ta,tb,out_dtype", [(0, 0, "bf16"), (0, 0, "fp32"), (1, 1, "fp32"), (0, 1, "bf16"),
                                             (1, 0, "bf16")])
def test_persistent_equals_one_workgroup_per_tile(ta, tb, out_dtype):
    """160 matrices of 264 x 296 are 640 tiles: the persistent launch gives each
    of the 256 work-groups two or three tiles (K = 200 and 1000 both end in a
    partial step), and must reproduce one work-group per tile bit for bit."""
    for m, n, k in [(264, 296, 200), (264, 296, 1000)]:
        idx = synth.sample_indices(7, 160, m, n, count=2048)
        outs = []
        for flags in (PERSIST, 0):
            got, ref, A, B, Cbuf = run(m, n, k, ta, tb, out_dtype, batch=160, seed=k + ta, flags=flags, idx=idx)
            outs.append(bits(Cbuf))
            check(got[idx[:, 0], idx[:, 1], idx[:, 2]], ref, tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)),
                  out_dtype, f"pingpong batch=160 m={m} n={n} k={k} flags={flags}")
        assert np.array_equal(outs[0], outs[1]), "persistent and per-tile launches differ"


def test_n_not_a_multiple_of_four():
    """B stored N x K lets N be odd; then the launch is not persistent and the
    last tile's columns are stored element by element."""
    idx = synth.sample_indices(8, 160, 264, 263, count=2048)
    got, ref, A, B, _ = run(264, 263, 136, 0, 1, "bf16", batch=160, seed=9, ldc_pad=1, idx=idx)
    check(got[idx[:, 0], idx[:, 1], idx[:, 2]], ref, tol_fp32(136, oracle.max_abs(A), oracle.max_abs(B)), "bf16",
          "pingpong n=263")


def test_k_zero_writes_zeros():
    # with A stored K x M and B stored K x N the vector loader accepts K = 0
    got, ref, *_ = run(264, 264, 0, 1, 0, "fp32")
    assert np.all(got == 0.0) and np.all(ref == 0.0)


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_epilogue_entry(out_dtype):
    """alpha/beta/bias through the ping-pong plan (the run call takes the
    epilogue entry), integer data: bit-exact."""
    rng = np.random.default_rng(21)
    m, n, k, batch = 264, 520, 200, 2
    A = synth.draw(rng, (batch, m, k), "int", -3, 3)
    B = synth.draw(rng, (batch, k, n), "int", -3, 3)
    tout = torch_out_dtype(out_dtype)
    if out_dtype == "fp32":
        C0 = rng.integers(-8, 9, size=(batch, m, n)).astype(np.float32)
        Cg = torch.from_numpy(C0.copy()).cuda()
        bv = rng.integers(-4, 5, size=n).astype(np.float32)
        bias_g = torch.from_numpy(bv).cuda()
        C0v, bias_v = C0.astype(np.float64), bv.astype(np.float64)
    else:
        cb = synth.draw(rng, (batch, m, n), "int", -8, 8, dtype=out_dtype)
        Cg = to_gpu(cb, out_dtype)
        bb = synth.draw(rng, (n,), "int", -4, 4, dtype=out_dtype)
        bias_g = to_gpu(bb, out_dtype)
        C0v, bias_v = oracle.decode(cb, out_dtype), oracle.decode(bb, out_dtype)
    pl = tg.plan(m, n, k, out_dtype=tout, batch=batch)
    pl = tg.plan_tile(pl, tg.VARIANT_TILE, tg.TILE_PINGPONG)
    tg.bmm_run_ex(pl, batch, m * k, k * n, m * n, to_gpu(A), to_gpu(B), Cg, alpha=2.0, beta=-1.0, bias=bias_g)
    torch.cuda.synchronize()
    P = oracle.gemm(A, B, m=m, n=n, k=k, batch=batch, stride_a=m * k, stride_b=k * n)
    ref = oracle.epilogue(P, 2.0, -1.0, C0v, bias_v)
    if out_dtype == "fp32":
        check_exact(values(Cg), ref, "fp32", "pingpong epilogue")
    else:
        check_exact(Cg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), ref, out_dtype,
                    "pingpong epilogue")


def test_planner_picks_it_for_the_large_square_product():
    pl = tg.plan(8192, 8192, 8192, out_dtype=torch.bfloat16)
    assert pl.variant == tg.VARIANT_TILE and pl.tile == tg.TILE_PINGPONG
