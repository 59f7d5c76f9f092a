"""Split-K products (gemm_splitk_run) against the oracle.

The parts of K run as one batched product (plus one product for a shorter
last part) into an fp32 workspace, then a fixed-order reduction writes C.
Covered here:
- every transpose, with uneven parts (the last part shorter);
- more splits than 8-element parts;
- M/N tails, including N not a multiple of 4 (scalar tail of the reduction);
- fp32 and 16-bit outputs, bf16 and fp16 inputs;
- integer inputs, which must match bit for bit and equal gemm_run bit for bit;
- repeat runs, which must be bitwise identical;
- K = 0 with no workspace;
- a long-K product at the suggested split count.
"""
import ctypes

import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
import synth
from parity import check, check_exact, to_gpu, tol_fp32, torch_out_dtype, values

pytestmark = pytest.mark.gpu

CANARY = -12345.0


def run(m, n, k, ta, tb, splits, out_dtype="fp32", in_dtype="bf16", seed=0, dist=("normal", 1.0), ldc_pad=0,
        idx=None):
    rng = np.random.default_rng(seed)
    ar, ac = (k, m) if ta else (m, k)
    br, bc = (n, k) if tb else (k, n)
    A = synth.draw(rng, (ar, ac), *dist, dtype=in_dtype)
    B = synth.draw(rng, (br, bc), *dist, dtype=in_dtype)
    tin = torch.bfloat16 if in_dtype == "bf16" else torch.float16
    tout = torch_out_dtype(out_dtype)
    ldc = n + ldc_pad
    Cbuf = torch.full((m, ldc), CANARY, dtype=tout, device="cuda")
    p = tg.plan(m, n, k, trans_a=ta, trans_b=tb, in_dtype=tin, out_dtype=tout, ldc=ldc)
    need = tg.splitk_workspace_bytes(p, splits)
    ws = torch.full(((need + 3) // 4 + 4,), float("nan"), dtype=torch.float32, device="cuda") if need else None
    Ag, Bg = to_gpu(A, in_dtype), to_gpu(B, in_dtype)
    tg.gemm_splitk_run(p, splits, ws, need, Ag, Bg, Cbuf)
    torch.cuda.synchronize()
    cb = values(Cbuf)
    canary = float(torch.tensor(CANARY, dtype=tout).item())
    assert np.all(cb[:, n:] == canary), "wrote into the ldc padding"
    ref = oracle.gemm(A[None], B[None], m=m, n=n, k=k, trans_a=ta, trans_b=tb, in_dtype=in_dtype, idx=idx)
    return cb[:, :n], ref, A, B, (Ag, Bg, Cbuf, p)


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_every_transpose(ta, tb, out_dtype):
    for i, (m, n, k, s) in enumerate([(256, 264, 4000, 4), (136, 72, 2056, 3), (16, 16, 24, 8), (200, 128, 1000, 7)]):
        got, ref, A, B, _ = run(m, n, k, ta, tb, s, out_dtype, seed=i, ldc_pad=8 * (i % 2))
        check(got, ref[0], tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), out_dtype,
              f"splitk m={m} n={n} k={k} splits={s} ta={ta} tb={tb} {out_dtype}")


def test_n_not_a_multiple_of_four():
    # B stored N x K lets the vector loader take N = 37; the reduction's last column group is partial
    got, ref, A, B, _ = run(72, 37, 1024, 0, 1, 4, "fp32", seed=5, ldc_pad=3)
    check(got, ref[0], tol_fp32(1024, oracle.max_abs(A), oracle.max_abs(B)), "fp32", "splitk n=37")


@pytest.mark.parametrize("out_dtype", ["fp32", "fp16"])
def test_fp16_inputs(out_dtype):
    got, ref, A, B, _ = run(128, 256, 3000, 0, 0, 5, out_dtype, in_dtype="fp16", seed=6)
    check(got, ref[0], tol_fp32(3000, oracle.max_abs(A, "fp16"), oracle.max_abs(B, "fp16")), out_dtype,
          "splitk fp16")


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_integer_inputs_bit_exact_and_equal_to_gemm_run(out_dtype):
    m, n, k = 192, 200, 4096
    got, ref, A, B, (Ag, Bg, Cbuf, p) = run(m, n, k, 1, 0, 6, out_dtype, seed=7, dist=("int", -4, 4))
    if out_dtype == "fp32":
        check_exact(got, ref[0], "fp32", "splitk int")
    else:
        check_exact(Cbuf.view(torch.int16).cpu().numpy().view(np.uint16), ref[0], "bf16", "splitk int bf16")
    C1 = torch.empty_like(Cbuf)
    tg.gemm_run(p, Ag, Bg, C1)
    torch.cuda.synchronize()
    assert torch.equal(C1, Cbuf), "split-K and gemm_run differ on exact sums"


def test_repeat_runs_are_bitwise_identical():
    rng = np.random.default_rng(8)
    m, n, k = 256, 256, 8192
    A = to_gpu(synth.draw(rng, (m, k), "normal", 1.0))
    B = to_gpu(synth.draw(rng, (k, n), "normal", 1.0))
    outs = [tg.gemm_splitk(A, B, splits=8) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_k_zero_writes_zeros_without_workspace():
    p = tg.plan(64, 64, 0)
    C = torch.full((64, 64), CANARY, dtype=torch.float32, device="cuda")
    a = torch.empty(8, dtype=torch.bfloat16, device="cuda")
    st = tg.lib().gemm_splitk_run(ctypes.byref(p), 4, None, 0, a.data_ptr(), a.data_ptr(), C.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK
    torch.cuda.synchronize()
    assert torch.all(C == 0)


def test_long_k_at_the_suggested_split():
    """1024 x 1024 x 65536, NN, bf16 out: 16 output tiles of 256 x 256, so the
    suggested split gives 16 parts (the batched product runs on the ping-pong
    kernel); sampled against the oracle."""
    m, n, k = 1024, 1024, 65536
    idx = synth.sample_indices(9, 1, m, n, count=1024)
    rng = np.random.default_rng(9)
    A = synth.draw(rng, (m, k), "normal", 1.0)
    B = synth.draw(rng, (k, n), "normal", 1.0)
    p = tg.plan(m, n, k, out_dtype=torch.bfloat16)
    assert tg.splitk_choose(p) == 16
    C = tg.gemm_splitk(to_gpu(A), to_gpu(B), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = values(C)[idx[:, 1], idx[:, 2]]
    ref = oracle.gemm(A[None], B[None], m=m, n=n, k=k, idx=idx)
    check(got, ref, tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), "bf16", "splitk 1024x1024x65536")
