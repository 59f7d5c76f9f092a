"""Edge cases of the HIP path through the C ABI: ragged M/N/K at tile
boundaries under all four transposes, padded leading dimensions whose padding
holds NaN (it must never leak into C), canaries around C (nothing outside the
M x N window may be written), misaligned bases (element-wise loader), K = 0,
integer inputs (bit-exact), every tile shape giving the same answer, fp16
inputs, and run-to-run determinism.

Boundary sizes follow the pages' advice to test shapes that are not tile
multiples, such as M = 17, 63, 129, and a tile larger than the problem
("Optimize Triton Block Parameters", Kernel design rules and Correctness
requirements).
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

NAN16 = np.uint16(0x7FC0)
CANARY = -12345.0
SIZES = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def padded(rng, rows, cols, ld, dist=("normal", 1.0), in_dtype="bf16"):
    """rows x cols matrix stored with leading dimension ld; padding is NaN."""
    X = np.full((rows, ld), NAN16 if in_dtype == "bf16" else np.uint16(0x7E00), dtype=np.uint16)
    X[:, :cols] = synth.draw(rng, (rows, cols), dist[0], *dist[1:], dtype=in_dtype)
    return X


def run_case(m, n, k, ta, tb, out_dtype="fp32", pad=(0, 0, 0), seed=0, dist=("normal", 1.0), in_dtype="bf16",
             variant=None, tile=None, offset_elems=0):
    rng = np.random.default_rng(seed)
    ar, ac = (k, m) if ta else (m, k)
    br, bc = (n, k) if tb else (k, n)
    lda, ldb, ldc = max(ac, 1) + pad[0], max(bc, 1) + pad[1], max(n, 1) + pad[2]
    A = padded(rng, ar, ac, lda, dist, in_dtype)
    B = padded(rng, br, bc, ldb, dist, in_dtype)
    tin = torch.bfloat16 if in_dtype == "bf16" else torch.float16
    tout = torch_out_dtype(out_dtype)
    # misaligned copies: the data starts offset_elems into a larger buffer
    Ag = to_gpu(np.concatenate([np.zeros(offset_elems, np.uint16), A.ravel()]), in_dtype)
    Bg = to_gpu(np.concatenate([np.zeros(offset_elems, np.uint16), B.ravel()]), in_dtype)
    rows_c = max(m, 1)
    Cbuf = torch.full((rows_c * ldc + 64 + offset_elems,), CANARY, dtype=tout, device="cuda")
    pl = tg.plan(m, n, k, trans_a=ta, trans_b=tb, in_dtype=tin, out_dtype=tout, lda=lda, ldb=ldb, ldc=ldc)
    if variant is not None:
        pl = tg.plan_tile(pl, variant, tile)
    st = tg.lib().gemm_run(ctypes.byref(pl), Ag.data_ptr() + 2 * offset_elems, Bg.data_ptr() + 2 * offset_elems,
                           Cbuf.data_ptr() + Cbuf.element_size() * offset_elems,
                           torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.status_str(st)
    torch.cuda.synchronize()
    cb = values(Cbuf)
    canary = float(torch.tensor(CANARY, dtype=tout).item())
    # everything outside the M x N window (ldc padding, tail, head) keeps its canary
    Cwin = cb[offset_elems:offset_elems + rows_c * ldc].reshape(rows_c, ldc)
    outside = np.concatenate([cb[:offset_elems], Cwin[:, n:].ravel(), cb[offset_elems + rows_c * ldc:]])
    assert np.all(outside == canary), "wrote outside C"
    ref = oracle.gemm(A, B, m=m, n=n, k=k, trans_a=ta, trans_b=tb, lda=lda, ldb=ldb, in_dtype=in_dtype)[0]
    got = Cwin[:m, :n]
    return got, ref, A, B, pl, Cbuf


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_ragged_boundaries_with_nan_padding(ta, tb, out_dtype):
    rng = np.random.default_rng(100 + 4 * ta + 2 * tb + (out_dtype == "bf16"))
    cases = [(17, 63, 129), (129, 17, 63), (64, 64, 48), (256, 256, 257), (1, 1, 1), (2, 255, 16)]
    cases += [tuple(int(x) for x in rng.choice(SIZES, 3)) for _ in range(10)]
    for i, (m, n, k) in enumerate(cases):
        pad = tuple(int(x) for x in rng.integers(0, 12, 3)) if i % 2 else (0, 0, 0)
        got, ref, A, B, pl, _ = run_case(m, n, k, ta, tb, out_dtype, pad=pad, seed=i)
        t = tol_fp32(k, oracle.max_abs(A[:, :A.shape[1] - pad[0]] if pad[0] else A),
                     oracle.max_abs(B[:, :B.shape[1] - pad[1]] if pad[1] else B))
        check(got, ref, t, out_dtype, f"m={m} n={n} k={k} ta={ta} tb={tb} pad={pad} variant={pl.variant}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_vector_path_tails_and_padding(ta, tb):
    """Shapes with every extent a multiple of 8 take the HBM->LDS vector loader."""
    for i, (m, n, k, pad) in enumerate([(264, 136, 72, (8, 16, 8)), (1000, 8, 40, (0, 0, 0)),
                                        (72, 1000, 1000, (8, 0, 24)), (520, 520, 8, (0, 8, 0))]):
        got, ref, A, B, pl, _ = run_case(m, n, k, ta, tb, "fp32", pad=pad, seed=50 + i)
        assert pl.variant == tg.VARIANT_TILE
        t = tol_fp32(k, oracle.max_abs(A[:, :A.shape[1] - pad[0]] if pad[0] else A),
                     oracle.max_abs(B[:, :B.shape[1] - pad[1]] if pad[1] else B))
        check(got, ref, t, "fp32", f"m={m} n={n} k={k} ta={ta} tb={tb}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_misaligned_base_takes_the_element_wise_loader(ta, tb):
    got, ref, A, B, pl, _ = run_case(96, 80, 64, ta, tb, "fp32", offset_elems=1, seed=7)
    check(got, ref, tol_fp32(64, oracle.max_abs(A), oracle.max_abs(B)), "fp32", "misaligned")


def test_k_zero_writes_zeros():
    got, ref, *_ = run_case(40, 24, 0, 0, 0, "fp32")
    assert np.all(got == 0.0) and np.all(ref == 0.0)


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_integer_inputs_are_bit_exact(out_dtype, ta, tb):
    for m, n, k in [(256, 256, 256), (1000, 1000, 1000), (16, 1024, 4096), (129, 65, 200)]:
        got, ref, *_ , Cbuf = run_case(m, n, k, ta, tb, out_dtype, dist=("int", -8, 8), seed=m + k)
        if out_dtype == "fp32":
            check_exact(got, ref, "fp32", f"int m={m} n={n} k={k}")
        else:
            raw = bits(Cbuf)[:m * n].reshape(m, n)
            check_exact(raw, ref, "bf16", f"int m={m} n={n} k={k}")


def test_every_tile_gives_the_same_answer():
    """Block parameters must never change the output: all tile shapes agree with
    the oracle, and bit for bit with each other on integer inputs."""
    shapes = [(v, t) for v in (tg.VARIANT_TILE, tg.VARIANT_GENERIC) for t in range(tg.variant_tiles(v))]
    for ta, tb in [(0, 0), (1, 1), (0, 1), (1, 0)]:
        ref_bits = None
        for variant, tile in shapes:
            got, ref, *_ = run_case(296, 264, 200, ta, tb, "fp32", dist=("int", -8, 8), seed=9,
                                    variant=variant, tile=tile)
            check_exact(got, ref, "fp32", f"variant={variant} tile={tile} ta={ta} tb={tb}")
            ref_bits = got if ref_bits is None else ref_bits
            assert np.array_equal(got, ref_bits)
        for variant, tile in shapes:
            got, ref, A, B, *_ = run_case(296, 264, 200, ta, tb, "fp32", seed=10, variant=variant, tile=tile)
            check(got, ref, tol_fp32(200, oracle.max_abs(A), oracle.max_abs(B)), "fp32",
                  f"variant={variant} tile={tile}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_kslice_uneven_k_splits(ta, tb):
    """The K-slice kernel gives wave w the K steps [w nk / 4, (w + 1) nk / 4):
    with one to three steps some waves get none, and a ragged last step is
    zero-filled; M and N end inside a tile.  Integer data with NaN padding:
    bit for bit, nothing written outside C.  (The kernel reads 16-byte units:
    extents and leading dimensions are multiples of 8.)"""
    cases = [(64, 64, 8), (72, 40, 16), (64, 200, 40), (136, 64, 96), (104, 96, 136), (256, 136, 200)]
    for i, (m, n, k) in enumerate(cases):
        pad = (8, 16, 8) if i % 2 else (0, 0, 0)
        got, ref, A, B, pl, _ = run_case(m, n, k, ta, tb, "fp32", pad=pad, seed=50 + i, dist=("int", -8, 8),
                                         variant=tg.VARIANT_TILE, tile=tg.TILE_KSLICE)
        assert pl.tile == tg.TILE_KSLICE
        check_exact(got, ref, "fp32", f"kslice m={m} n={n} k={k} ta={ta} tb={tb} pad={pad}")


def test_skinny_variants_and_tails():
    assert tg.variant_tiles(tg.VARIANT_SKINNY) == 2
    cases = [(0, 16), (0, 5), (1, 32), (1, 17)]
    for tile, m in cases:
        # K of only a few stages makes most ring refills read out of range
        # (they return zeros at once): the refill must not overtake another
        # wave's reads of the buffer it overwrites
        for n, k in [(8192, 1024), (4096, 512), (100, 1000), (33, 8)]:
            got, ref, A, B, pl, _ = run_case(m, n, k, 0, 1, "bf16", seed=tile + n, variant=tg.VARIANT_SKINNY,
                                             tile=tile)
            check(got, ref, tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), "bf16",
                  f"skinny tile={tile} m={m} n={n} k={k}")


@pytest.mark.parametrize("out_dtype", ["fp32", "fp16"])
def test_fp16_inputs(out_dtype):
    for ta, tb in [(0, 0), (1, 1), (0, 1)]:
        for m, n, k in [(256, 256, 256), (17, 129, 63), (16, 512, 512)]:
            got, ref, A, B, *_ = run_case(m, n, k, ta, tb, out_dtype, in_dtype="fp16", seed=m)
            check(got, ref, tol_fp32(k, oracle.max_abs(A, "fp16"), oracle.max_abs(B, "fp16")), out_dtype,
                  f"fp16 m={m} n={n} k={k}")


def test_repeated_runs_are_bitwise_identical():
    (p,) = synth.square_256()
    A, B = to_gpu(p.A), to_gpu(p.B)
    outs = [tg.gemm(A, B) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_batched_broadcast_and_strides():
    rng = np.random.default_rng(3)
    batch, m, n, k = 5, 130, 72, 96
    A = synth.draw(rng, (batch, m, k), "normal", 1.0)
    B = synth.draw(rng, (k, n), "normal", 1.0)   # one B for every batch (stride 0)
    Ag, Bg = to_gpu(A), to_gpu(B)
    C = torch.full((batch, m, n), CANARY, device="cuda")
    pl = tg.plan(m, n, k)
    tg.bmm_run(pl, batch, m * k, 0, m * n, Ag, Bg, C)
    torch.cuda.synchronize()
    ref = oracle.gemm(A, B, m=m, n=n, k=k, batch=batch, stride_a=m * k, stride_b=0)
    check(values(C), ref, tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B)), "fp32", "broadcast B")


@pytest.mark.parametrize("ta,tb,out_dtype", [(0, 0, "fp32"), (1, 1, "fp32"), (0, 1, "fp32"), (0, 1, "bf16")])
def test_persistent_launch_matches_one_workgroup_per_tile(ta, tb, out_dtype):
    """Persistent work-groups (each loops over tiles; with PREFETCH the next
    tile's first copies are issued before this tile's stores) compute exactly what one
    work-group per tile computes -- the K walk and the summation order are the
    same -- on ragged batched shapes with enough tiles that the launcher does
    loop, with a masked K tail and with a K of several ring lengths."""
    rng = np.random.default_rng(77)
    tout = torch_out_dtype(out_dtype)
    # 160 matrices of 264 x 264: >= 2 items per resident work-group for every tile below
    # (e.g. 4 256x256 tiles x 160 = 640 > 2 x 256), so the launcher does loop
    for (m, n, k, batch) in [(264, 264, 96, 160), (264, 264, 1000, 160)]:
        ar, ac = (k, m) if ta else (m, k)
        br, bc = (n, k) if tb else (k, n)
        A = synth.draw(rng, (batch, ar, ac), "normal", 1.0)
        B = synth.draw(rng, (batch, br, bc), "normal", 1.0)
        Ag, Bg = to_gpu(A), to_gpu(B)
        base = tg.plan(m, n, k, trans_a=ta, trans_b=tb, out_dtype=tout, batch=batch)
        idx = synth.sample_indices(5, batch, m, n, count=2048)
        ref = oracle.gemm(A, B, m=m, n=n, k=k, trans_a=ta, trans_b=tb, batch=batch, stride_a=ar * ac,
                          stride_b=br * bc, idx=idx)
        t = tol_fp32(k, oracle.max_abs(A), oracle.max_abs(B))
        # every tile-kernel entry the planner or the grouped launch uses for these shapes
        for tile in (0, 1, 3, 4, 11):
            outs = []
            both = tg.FLAG_PERSIST | tg.FLAG_PREFETCH
            for flags in (both, tg.FLAG_PERSIST, 0):
                pl = tg.plan_tile(base, tg.VARIANT_TILE, tile)
                pl.flags = (pl.flags & ~both) | flags
                C = torch.full((batch, m, n), CANARY, dtype=tout, device="cuda")
                tg.bmm_run(pl, batch, ar * ac, br * bc, m * n, Ag, Bg, C)
                torch.cuda.synchronize()
                outs.append((bits(C), values(C)))
            what = f"persistent tile={tile} m={m} n={n} k={k} batch={batch} ta={ta} tb={tb} out={out_dtype}"
            for o in outs[1:]:
                assert np.array_equal(outs[0][0], o[0]), what
            got = outs[0][1][idx[:, 0], idx[:, 1], idx[:, 2]]
            check(got, ref, t, out_dtype, what)


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_non_temporal_c_stores_give_the_same_result(out_dtype):
    """TG_FLAG_STREAM_C only changes the cache policy of the C stores."""
    rng = np.random.default_rng(31)
    m, n, k, batch = 264, 392, 200, 3
    A = to_gpu(synth.draw(rng, (batch, m, k), "normal", 1.0))
    B = to_gpu(synth.draw(rng, (batch, n, k), "normal", 1.0))
    tout = torch_out_dtype(out_dtype)
    outs = []
    for flag in (0, 1):
        p = tg.plan(m, n, k, trans_b=True, out_dtype=tout, batch=batch)
        p.flags = (p.flags & ~tg.FLAG_STREAM_C) | (tg.FLAG_STREAM_C if flag else 0)
        C = torch.empty((batch, m, n), dtype=tout, device="cuda")
        tg.bmm_run(p, batch, m * k, n * k, m * n, A, B, C)
        outs.append(C)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
