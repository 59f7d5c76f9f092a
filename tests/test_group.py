"""Grouped launches (gemm_group_run): many products of different shapes in one
grid, checked problem by problem against the oracle with the GEMM tolerance
(parity.py), bit for bit on integer-valued inputs, under all four transposes,
every group tile, both output types, and the edge cases of the call: empty
problems, K = 0, more problems than one launch holds, problems the vector
loader cannot serve, and output padding that must keep its canaries."""
import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
import synth
from parity import check, check_exact, to_gpu, tol_fp32, torch_out_dtype, values

pytestmark = pytest.mark.gpu

CANARY = -12288.0  # exact in fp32, bf16 and fp16
# ragged shapes: tile edges, thin and empty problems, K = 0
SHAPES = [(1, 8, 8), (17, 33, 64), (64, 64, 64), (65, 129, 72), (128, 8, 256), (200, 96, 40), (0, 64, 64),
          (64, 0, 64), (96, 64, 0), (256, 320, 128), (33, 256, 1000), (512, 136, 64)]


def make(rng, m, n, k, ta, tb, in_dtype, dist, pad_c=0):
    ar, ac = (k, m) if ta else (m, k)
    br, bc = (n, k) if tb else (k, n)
    A = synth.draw(rng, (ar, ac), *dist, dtype=in_dtype)
    B = synth.draw(rng, (br, bc), *dist, dtype=in_dtype)
    return A, B, max(n, 1) + pad_c


def run_group(shapes, ta, tb, in_dtype="bf16", out_dtype="fp32", tile=-1, seed=0, dist=("normal", 1.0), pad_c=0,
              exact=False):
    rng = np.random.default_rng(seed)
    tin = torch.bfloat16 if in_dtype == "bf16" else torch.float16
    tout = torch_out_dtype(out_dtype)
    probs, host, outs = [], [], []
    for (m, n, k) in shapes:
        A, B, ldc = make(rng, m, n, k, ta, tb, in_dtype, dist, pad_c)
        Ag, Bg = to_gpu(A, in_dtype), to_gpu(B, in_dtype)
        C = torch.full((max(m, 1), ldc), CANARY, dtype=tout, device="cuda")
        lda = max(A.shape[1], 1)
        ldb = max(B.shape[1], 1)
        probs.append((m, n, k, lda, ldb, ldc, Ag, Bg, C))
        host.append((A, B, lda, ldb))
        outs.append(C)
    tg.gemm_group_run(tg._dtype_code(tin), tg._dtype_code(tout), ta, tb, probs, tile)
    torch.cuda.synchronize()
    for (m, n, k), (A, B, lda, ldb), C in zip(shapes, host, outs):
        what = f"group {m}x{n}x{k} ta={ta} tb={tb} {in_dtype}->{out_dtype} tile={tile}"
        got = values(C)
        if m == 0 or n == 0:
            assert np.all(got == CANARY), f"{what}: empty problem wrote output"
            continue
        assert np.all(got[:m, n:] == CANARY), f"{what}: wrote past column n"
        ref = oracle.gemm(A, B, m=m, n=n, k=k, trans_a=ta, trans_b=tb, lda=lda, ldb=ldb, in_dtype=in_dtype)[0]
        if exact:
            if out_dtype == "fp32":
                check_exact(got[:m, :n], ref, out_dtype, what)
            else:
                bits = C[:m, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                check_exact(bits, ref, out_dtype, what)
        else:
            t = tol_fp32(k, oracle.max_abs(A, in_dtype), oracle.max_abs(B, in_dtype)) if k else 0.0
            check(got[:m, :n], ref, t, out_dtype, what)


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("tile", [-1, 0, 1, 2, 3, 4, 5, 6])
def test_group_matches_oracle(ta, tb, tile):
    print(f"group ta={ta} tb={tb} tile={tile}", flush=True)
    run_group(SHAPES, ta, tb, tile=tile, seed=10 * ta + tb + tile + 2)


@pytest.mark.parametrize("in_dtype,out_dtype", [("bf16", "bf16"), ("fp16", "fp32"), ("fp16", "fp16")])
def test_group_dtypes(in_dtype, out_dtype):
    run_group(SHAPES, 0, 1, in_dtype=in_dtype, out_dtype=out_dtype, seed=5)


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_group_integer_inputs_bit_exact(tile, out_dtype):
    """Small integers: every partial sum is exact in fp32, so every tile and
    summation order must give the oracle's value exactly."""
    run_group(SHAPES, 1, 0, out_dtype=out_dtype, tile=tile, seed=7, dist=("int", -4, 4), exact=True)


def test_group_more_problems_than_one_launch_holds():
    rng = np.random.default_rng(3)
    shapes = [(int(m), int(n), int(k)) for m, n, k in zip(rng.integers(1, 300, 70), rng.integers(8, 300, 70) // 8 * 8,
                                                          rng.integers(8, 200, 70) // 8 * 8)]
    run_group(shapes, 0, 0, seed=4, pad_c=8)


def test_group_falls_back_for_unaligned_problems():
    """A problem with an odd leading dimension cannot use the vector loader; it
    runs through the element-wise kernel in the same call."""
    shapes = [(64, 64, 64), (31, 33, 35), (128, 64, 96)]
    run_group(shapes, 0, 0, seed=8)


def test_group_matches_single_launches_on_integers():
    """The grouped kernel and gemm_run agree bit for bit where sums are exact."""
    rng = np.random.default_rng(11)
    shapes = [(200, 136, 96), (64, 512, 128), (300, 40, 264)]
    tin = torch.bfloat16
    for (m, n, k) in shapes:
        A = to_gpu(synth.draw(rng, (m, k), "int", -3, 3))
        B = to_gpu(synth.draw(rng, (k, n), "int", -3, 3))
        (Cg,) = tg.gemm_group([A], [B], out_dtype=torch.float32)
        Cs = tg.gemm(A, B, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(Cg, Cs), (m, n, k)
        assert A.dtype == tin


def test_grouped_moe_workload_sampled():
    """The grouped-launch workload at its full size (32 ragged experts over
    8192 token rows, K = N = 1024, bf16 out), launched as the benchmark does
    -- one table whose problems are row ranges of X and Y -- and checked on a
    sample of each expert's outputs (tile edges included) against the oracle.
    Rows outside every expert's range keep their canary."""
    p = synth.grouped_moe()
    T = int(p.counts.sum())
    off = p.offsets
    Xg, Wg = to_gpu(p.X), to_gpu(p.W)
    Y = torch.full((T + 8, p.n), CANARY, dtype=torch.bfloat16, device="cuda")
    probs = []
    for e, c in enumerate(p.counts):
        c = int(c)
        probs.append((c, p.n, p.k, p.k, p.n, p.n, Xg[int(off[e]):int(off[e]) + c], Wg[e],
                      Y[int(off[e]):int(off[e]) + c]))
    tg.gemm_group_run(tg.TG_BF16, tg.TG_BF16, False, False, probs)
    torch.cuda.synchronize()
    got_all = values(Y)
    assert np.all(got_all[T:] == CANARY), "wrote past the last expert's rows"
    rng = np.random.default_rng(77)
    t = tol_fp32(p.k, oracle.max_abs(p.X), oracle.max_abs(p.W))
    for e, c in enumerate(p.counts):
        c = int(c)
        if c == 0:
            continue
        rows = np.unique(np.concatenate([rng.integers(0, c, 96), [0, c - 1, min(c - 1, 127), min(c - 1, 128)]]))
        cols = rng.integers(0, p.n, rows.size)
        cols[:2] = [0, p.n - 1]
        idx = np.stack([np.zeros_like(rows), rows, cols], axis=1)
        X_e = np.ascontiguousarray(p.X[int(off[e]):int(off[e]) + c])
        ref = oracle.gemm(X_e, p.W[e], m=c, n=p.n, k=p.k, idx=idx)
        got = got_all[int(off[e]) + rows, cols]
        check(got, ref, t, "bf16", f"expert {e} ({c} rows)")
