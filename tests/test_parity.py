"""HIP path vs the CPU oracle on the five workloads, element by element.

Small and medium problems are compared in full; the full-size batched and
8192^3 products are compared on 4096 seeded samples plus tile-edge points
(the oracle computes each sampled element from the definition).  Tolerances
are the ones in tests/parity.py.  Every call goes through the C ABI
(gemm_plan / gemm_run / bmm_run) in the launch configuration the planner
picks, the same one the benchmark times.
"""
import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
import synth
from parity import bits, check, check_exact, to_gpu, tol_fp32, torch_out_dtype, values

pytestmark = pytest.mark.gpu


def run(p: synth.Problem, out_dtype: str = None, A=None, B=None):
    out_dtype = out_dtype or p.out_dtype
    A = to_gpu(p.A, p.in_dtype) if A is None else A
    B = to_gpu(p.B, p.in_dtype) if B is None else B
    pl = tg.plan(p.m, p.n, p.k, trans_a=p.trans_a, trans_b=p.trans_b,
                 in_dtype=torch.bfloat16 if p.in_dtype == "bf16" else torch.float16,
                 out_dtype=torch_out_dtype(out_dtype), lda=p.lda, ldb=p.ldb, ldc=p.ldc)
    if p.batch == 1:
        C = torch.empty((p.m, p.n), dtype=torch_out_dtype(out_dtype), device="cuda")
        tg.gemm_run(pl, A, B, C)
    else:
        C = torch.empty((p.batch, p.m, p.n), dtype=torch_out_dtype(out_dtype), device="cuda")
        tg.bmm_run(pl, p.batch, p.stride_a, p.stride_b, p.stride_c, A, B, C)
    torch.cuda.synchronize()
    return C, pl


def tolerance(p: synth.Problem) -> float:
    return tol_fp32(p.k, oracle.max_abs(p.A, p.in_dtype), oracle.max_abs(p.B, p.in_dtype))


def compare_full(p, out_dtype=None):
    out_dtype = out_dtype or p.out_dtype
    C, pl = run(p, out_dtype)
    ref = oracle.gemm_problem(p)
    got = values(C).reshape(ref.shape)
    r = check(got, ref, tolerance(p), out_dtype, p.name)
    print(f"{p.name} out={out_dtype} variant={pl.variant} tile={pl.bm}x{pl.bn}x{pl.bk} worst err/bound={r:.3f}")
    return C


def compare_sampled(p, out_dtype=None, seed=0, C=None):
    out_dtype = out_dtype or p.out_dtype
    if C is None:
        C, pl = run(p, out_dtype)
    idx = synth.sample_indices(seed, p.batch, p.m, p.n)
    ref = oracle.gemm_problem(p, idx=idx)
    Cv = C.reshape(p.batch, p.m, p.n)
    ii = torch.from_numpy(idx).cuda()
    got = Cv[ii[:, 0], ii[:, 1], ii[:, 2]].to(torch.float64).cpu().numpy()
    r = check(got, ref, tolerance(p), out_dtype, p.name)
    print(f"{p.name} out={out_dtype} sampled {len(idx)} worst err/bound={r:.3f}")
    return C


def test_square_256():
    (p,) = synth.square_256()
    compare_full(p)


@pytest.mark.parametrize("combo", range(4))
def test_ragged_1000_every_transpose(combo):
    p = synth.ragged_1000()[combo]
    compare_full(p)


def test_skinny_16_bf16_out_and_fp32_out():
    (p,) = synth.skinny_16()
    compare_full(p, "bf16")
    compare_full(p, "fp32")


@pytest.fixture(scope="module")
def attention():
    return synth.attention_bmm()


def test_attention_scores_full_size_sampled(attention):
    s, _ = attention
    C = compare_sampled(s)
    assert torch.isfinite(C).all().item()


def test_attention_output_full_size_sampled(attention):
    _, o = attention
    C = compare_sampled(o)
    assert torch.isfinite(C).all().item()


def test_attention_reduced_batch_full():
    for p in synth.attention_bmm(seed=30, batch=3, seq=384, head=128):
        compare_full(p)


def test_square_8192_sampled_bf16_and_fp32():
    (p,) = synth.square_8192()
    C = compare_sampled(p, "bf16", seed=4)
    assert torch.isfinite(C.float()).all().item()
    del C
    compare_sampled(p, "fp32", seed=5)
