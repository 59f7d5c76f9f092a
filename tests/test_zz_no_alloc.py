"""gemm_splitk_run_noalloc: split-K with the library's fixed per-device
scratch array instead of a caller workspace.

Through the C ABI, two calls in a row on one GPU -- the second smaller, so it
reuses the array the first one filled -- each compared with gemm_splitk_run
on a caller workspace (same plan, same split: the same parts and the same
order of additions, so the outputs must be bit-identical) and with the
oracle (the acceptance rule of the other parity tests).  Sizes beyond the
array are refused before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
import synth
from parity import bits, check, to_gpu, tol_fp32, torch_out_dtype, values

pytestmark = pytest.mark.gpu

CANARY = -12345.0


def _call_both(m, n, k, ta, tb, splits, out_dtype, seed, ldc_pad=0):
    rng = np.random.default_rng(seed)
    ar, ac = (k, m) if ta else (m, k)
    br, bc = (n, k) if tb else (k, n)
    A = synth.draw(rng, (ar, ac), "normal", 1.0)
    B = synth.draw(rng, (br, bc), "normal", 1.0)
    tout = torch_out_dtype(out_dtype)
    ldc = n + ldc_pad
    p = tg.plan(m, n, k, trans_a=ta, trans_b=tb, out_dtype=tout, ldc=ldc)
    need = tg.splitk_workspace_bytes(p, splits)
    assert 0 < need <= tg.SPLITK_SCRATCH_BYTES
    Ag, Bg = to_gpu(A), to_gpu(B)
    C_ws = torch.full((m, ldc), CANARY, dtype=tout, device="cuda")
    C_na = torch.full((m, ldc), CANARY, dtype=tout, device="cuda")
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    L = tg.lib()
    stream = torch.cuda.current_stream().cuda_stream
    print(f"noalloc case m={m} n={n} k={k} ta={ta} tb={tb} splits={splits} {out_dtype}", flush=True)
    st = L.gemm_splitk_run(ctypes.byref(p), splits, ws.data_ptr(), need, Ag.data_ptr(), Bg.data_ptr(),
                           C_ws.data_ptr(), stream)
    assert st == tg.TG_OK, tg.status_str(st)
    st = L.gemm_splitk_run_noalloc(ctypes.byref(p), splits, Ag.data_ptr(), Bg.data_ptr(), C_na.data_ptr(), stream)
    assert st == tg.TG_OK, tg.status_str(st)
    torch.cuda.synchronize()
    return A, B, C_ws, C_na


def _compare(m, n, k, ta, tb, splits, out_dtype, seed, ldc_pad=0, sample=None):
    A, B, C_ws, C_na = _call_both(m, n, k, ta, tb, splits, out_dtype, seed, ldc_pad)
    what = f"noalloc m={m} n={n} k={k} splits={splits} {out_dtype}"
    assert np.array_equal(bits(C_na) if out_dtype != "fp32" else C_na.cpu().numpy().view(np.uint32),
                          bits(C_ws) if out_dtype != "fp32" else C_ws.cpu().numpy().view(np.uint32)), \
        f"{what}: differs from gemm_splitk_run with a caller workspace"
    got = values(C_na)
    canary = float(torch.tensor(CANARY, dtype=torch_out_dtype(out_dtype)).item())
    assert np.all(got[:, n:] == canary), f"{what}: wrote into the ldc padding"
    t = tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B))
    if sample is None:
        ref = oracle.gemm(A[None], B[None], m=m, n=n, k=k, trans_a=ta, trans_b=tb)[0]
        check(got[:, :n], ref, t, out_dtype, what)
    else:
        rng = np.random.default_rng(1234)
        idx = np.stack([np.zeros(sample, np.int64), rng.integers(0, m, sample), rng.integers(0, n, sample)], 1)
        ref = oracle.gemm(A[None], B[None], m=m, n=n, k=k, trans_a=ta, trans_b=tb, idx=idx)
        check(got[idx[:, 1], idx[:, 2]], ref, t, out_dtype, what)


def test_two_calls_in_a_row_second_smaller():
    # 1024 x 1024 x 65536 in 16 parts fills the array exactly (16 x 1024 x 1024 fp32 = 64 MiB)
    _compare(1024, 1024, 65536, 0, 0, 16, "bf16", seed=21, sample=4096)
    # then a smaller ragged product with a shorter last part, transposed operands and fp32 output
    _compare(200, 136, 3000, 1, 1, 5, "fp32", seed=22, ldc_pad=8)


def test_sizes_beyond_the_array_are_refused():
    p = tg.plan(1024, 1032, 65536)  # 16 parts of 1024 x 1032 floats: just over 64 MiB
    assert tg.splitk_workspace_bytes(p, 16) > tg.SPLITK_SCRATCH_BYTES
    A = ctypes.c_void_p(1 << 20)  # never dereferenced: the size check comes first
    st = tg.lib().gemm_splitk_run_noalloc(ctypes.byref(p), 16, A, A, A, None)
    assert st == tg.TG_ERR_TOO_LARGE
    assert "scratch" in tg.status_str(st)
