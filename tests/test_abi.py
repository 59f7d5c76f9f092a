"""The C-ABI library without a GPU: it loads, exports every declared symbol,
its plan struct matches the header, and gemm_plan()/the run-time argument
checks behave as include/tgemm.h documents.  No kernel is launched here."""
import ctypes
import json
import os
import re
import shutil
import subprocess

import pytest

import matmul_tiled_bf16_amd as tg
from matmul_tiled_bf16_amd import roofline

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgemm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"gemm_plan", "bmm_plan", "gemm_plan_tile", "gemm_run", "bmm_run", "tg_status_str", "tg_abi_version",
            "tg_variant_tiles", "attention_fwd", "gemm_group_run", "tg_group_tiles", "gemm_splitk_run",
            "tg_splitk_workspace_bytes", "tg_splitk_choose"} <= set(names)
    L = tg.lib()
    for n in names:
        assert hasattr(L, n), f"libtgemm.so does not export {n}"
    nm = subprocess.run(["nm", "-D", "--defined-only", tg.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), f"{n} not a defined text symbol"


def test_abi_version_matches_header():
    assert tg.lib().tg_abi_version() == tg._abi_version_from_header()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plan_struct_layout_matches_header(tmp_path):
    fields = [f for f, _ in tg.GemmPlan._fields_]
    prog = ['#include <stdio.h>', '#include <stddef.h>', '#include "tgemm.h"', 'int main(void) {',
            'printf("%zu\\n", sizeof(gemm_plan_t));']
    prog += [f'printf("%zu\\n", offsetof(gemm_plan_t, {f}));' for f in fields]
    prog += ['return 0; }']
    c = tmp_path / "layout.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.dirname(HEADER)}", "-I/opt/rocm/include",
                        str(c), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("the HIP runtime header does not compile with plain gcc here: " + r.stderr[-300:])
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(tg.GemmPlan)
    for f, off in zip(fields, out[1:]):
        assert getattr(tg.GemmPlan, f).offset == off, f


def test_variant_tile_counts():
    counts = [tg.variant_tiles(v) for v in (tg.VARIANT_GENERIC, tg.VARIANT_TILE, tg.VARIANT_SKINNY)]
    assert all(c >= 1 for c in counts)
    assert tg.variant_tiles(7) == 0 and tg.variant_tiles(-1) == 0
    # the last valid index of each variant passes the launcher's re-validation; one past it does not
    st, p = raw_plan(m=64, n=64, k=64)
    for v, c in zip((tg.VARIANT_GENERIC, tg.VARIANT_TILE), counts[:2]):
        q = tg.GemmPlan.from_buffer_copy(p)
        q.variant, q.tile = v, c
        assert tg.lib().gemm_run(ctypes.byref(q), 16, 16, 16, None) == tg.TG_ERR_UNSUPPORTED


def test_plan_tile_rederives_the_plan():
    st, p = raw_plan(m=2048, n=128, k=2048)
    assert st == tg.TG_OK
    q = tg.plan_tile(p, tg.VARIANT_TILE, 1)          # 128 x 128: one column of tiles
    assert (q.variant, q.tile, q.bm, q.bn, q.tiles_m, q.tiles_n) == (tg.VARIANT_TILE, 1, 128, 128, 16, 1)
    assert q.flags & tg.FLAG_ROTATE_K and q.flags & tg.FLAG_EVEN_K
    assert q.lds_bytes == roofline.lds_budget(128, 128, q.bk, q.stages)
    r = tg.plan_tile(q, tg.VARIANT_GENERIC, 0)
    assert r.variant == tg.VARIANT_GENERIC and not r.flags & tg.FLAG_ROTATE_K
    L = tg.lib()
    bad = tg.GemmPlan.from_buffer_copy(p)
    for variant, tile in [(tg.VARIANT_TILE, tg.variant_tiles(tg.VARIANT_TILE)), (tg.VARIANT_SKINNY, 0), (9, 0)]:
        assert L.gemm_plan_tile(ctypes.byref(bad), variant, tile) == tg.TG_ERR_UNSUPPORTED
        assert bytes(bad) == bytes(p), "a failed re-plan leaves the plan unchanged"
    stale = tg.GemmPlan.from_buffer_copy(p)
    stale.abi_version = 0
    assert L.gemm_plan_tile(ctypes.byref(stale), tg.VARIANT_TILE, 0) == tg.TG_ERR_INVALID
    assert L.gemm_plan_tile(None, tg.VARIANT_TILE, 0) == tg.TG_ERR_INVALID


def test_status_strings():
    assert tg.status_str(tg.TG_OK) == "ok"
    assert tg.status_str(tg.TG_ERR_INVALID) == "invalid argument"
    assert tg.status_str(tg.TG_ERR_UNSUPPORTED) == "unsupported"
    assert tg.status_str(tg.TG_ERR_HIP) == "HIP launch error"
    assert tg.status_str(99) == "unknown status"


def raw_plan(in_t=0, out_t=2, ta=0, tb=0, m=64, n=64, k=64, lda=None, ldb=None, ldc=None):
    p = tg.GemmPlan()
    lda = lda if lda is not None else max(1, m if ta else k)
    ldb = ldb if ldb is not None else max(1, k if tb else n)
    ldc = ldc if ldc is not None else max(1, n)
    st = tg.lib().gemm_plan(ctypes.byref(p), in_t, out_t, ta, tb, m, n, k, lda, ldb, ldc)
    return st, p


@pytest.mark.parametrize("kw,status", [
    (dict(m=-1), tg.TG_ERR_INVALID),
    (dict(k=-5), tg.TG_ERR_INVALID),
    (dict(ta=2), tg.TG_ERR_INVALID),
    (dict(tb=-1), tg.TG_ERR_INVALID),
    (dict(m=64, k=100, lda=99), tg.TG_ERR_INVALID),          # lda < K
    (dict(ta=1, m=100, k=64, lda=99), tg.TG_ERR_INVALID),    # transposed A: lda < M
    (dict(n=100, ldb=99), tg.TG_ERR_INVALID),
    (dict(tb=1, k=100, ldb=99), tg.TG_ERR_INVALID),
    (dict(n=100, ldc=99), tg.TG_ERR_INVALID),
    (dict(m=1 << 31), tg.TG_ERR_INVALID),
    (dict(in_t=2), tg.TG_ERR_UNSUPPORTED),                    # fp32 inputs
    (dict(in_t=1, out_t=0), tg.TG_ERR_UNSUPPORTED),           # fp16 -> bf16
    (dict(in_t=0, out_t=1), tg.TG_ERR_UNSUPPORTED),           # bf16 -> fp16
    (dict(in_t=0, out_t=0), tg.TG_OK),
    (dict(in_t=1, out_t=1), tg.TG_OK),
    (dict(in_t=1, out_t=2), tg.TG_OK),
    (dict(m=0, n=0, k=0), tg.TG_OK),
])
def test_plan_validation(kw, status):
    st, p = raw_plan(**kw)
    assert st == status
    if st != tg.TG_OK:
        assert p.abi_version != tg._abi_version_from_header(), "failed plan must not look valid"


def test_null_plan_pointer():
    assert tg.lib().gemm_plan(None, 0, 2, 0, 0, 1, 1, 1, 1, 1, 1) == tg.TG_ERR_INVALID
    assert tg.lib().gemm_run(None, None, None, None, None) == tg.TG_ERR_INVALID
    assert tg.lib().bmm_run(None, 1, 0, 0, 0, None, None, None, None) == tg.TG_ERR_INVALID


def test_plan_choices_for_the_workloads():
    # 256^3 NN fp32 out: too few 128-tiles to fill 256 CUs -> 64x64 tiles, K multiple of 64
    p = tg.plan(256, 256, 256)
    assert (p.variant, p.bm, p.bn, p.flags & tg.FLAG_EVEN_K, p.flags & tg.FLAG_VEC16) == (
        tg.VARIANT_TILE, 64, 64, tg.FLAG_EVEN_K, tg.FLAG_VEC16)
    assert (p.tile, p.stages) == (12, 4)  # 16 tiles: their four waves split K
    # 1000^3, every transpose: vector path (1000 = 8*125), ragged K tail
    for ta in (0, 1):
        for tb in (0, 1):
            p = tg.plan(1000, 1000, 1000, trans_a=ta, trans_b=tb)
            assert p.variant == tg.VARIANT_TILE and p.flags & tg.FLAG_VEC16 and not p.flags & tg.FLAG_EVEN_K
            assert (p.tile, p.bm, p.bn, p.stages) == (12, 64, 64, 4)  # 256 tiles, one per CU: K split 4 ways
            assert p.tiles_m * p.tiles_n >= 64
    # skinny M = 16, B stored N x K
    import torch
    p = tg.plan(16, 8192, 8192, trans_b=True, out_dtype=torch.bfloat16)
    assert p.variant == tg.VARIANT_SKINNY and p.bm >= 16
    # attention-shaped batched products and the big square GEMM
    p = tg.plan(2048, 2048, 128, trans_b=True)
    assert p.variant == tg.VARIANT_TILE and p.flags & tg.FLAG_EVEN_K
    p = tg.plan(2048, 128, 2048)
    assert p.variant == tg.VARIANT_TILE
    # batched attention shapes, planned for their batch of 128 (HBM-bound): 128x128 tiles for S,
    # 256x128 for the single-column O = P V, which rotates its K walks
    for mm, nn, kk, tb in [(2048, 2048, 128, True), (2048, 128, 2048, False)]:
        p = tg.plan(mm, nn, kk, trans_b=tb, batch=128)
        assert (p.variant, p.bm, p.bn) == (tg.VARIANT_TILE, 256 if nn == 128 else 128, 128)
        assert bool(p.flags & tg.FLAG_ROTATE_K) == (nn == 128)
        assert p.flags & tg.FLAG_PERSIST and not p.flags & tg.FLAG_PREFETCH  # HBM-bound: LDS-staged stores
        assert p.flags & tg.FLAG_STREAM_C  # outputs of 128 MiB and 2 GiB: non-temporal stores
        assert tg.plan_tile(p, tg.VARIANT_TILE, 1).flags & tg.FLAG_STREAM_C  # kept by a re-plan
    assert not tg.plan(2048, 2048, 128, trans_b=True).flags & tg.FLAG_STREAM_C  # 16 MiB: stays cached
    # short K with many tiles: the panel kernel (A stored M x K); A stored K x M, a long K, or too few
    # tiles keep the 128 x 128 tile kernel
    assert tg.plan(2048, 2048, 128, trans_b=True, batch=128).tile == tg.TILE_PANEL
    assert tg.plan(2048, 2048, 64, batch=128, out_dtype=torch.bfloat16).tile == tg.TILE_PANEL
    assert tg.plan(2048, 2048, 128, trans_a=True, trans_b=True, batch=128).tile == 4
    assert tg.plan(2048, 2048, 136, trans_b=True, batch=128).tile == 4
    assert tg.plan(2048, 2048, 128, trans_b=True).tile == 4
    assert tg.plan(2048, 128, 2048, batch=128).tile == 17                      # N <= 256: 256 x 128
    assert tg.plan(2048, 64, 2048, batch=128, out_dtype=torch.bfloat16).tile == 17
    assert tg.plan(16384, 128, 16384).tile != 17                                # 64 of its items
    assert tg.plan(2048, 512, 2048, batch=128).tile == 4                        # N > 256
    with pytest.raises(tg.TgError):
        tg.plan(64, 64, 64, batch=0)
    p = tg.plan(8192, 8192, 8192, out_dtype=torch.bfloat16)
    assert (p.variant, p.bm, p.bn, p.wg_threads) == (tg.VARIANT_TILE, 256, 256, 512) and p.tiles_m * p.tiles_n == 1024
    # MFMA-bound products take the ping-pong kernel above 128 of its 256 x 256 work items,
    # the 128 x 128 tile with two work-groups per CU below
    assert tg.plan(3072, 3072, 8192, out_dtype=torch.bfloat16).tile == tg.TILE_PINGPONG  # 144 items
    assert tg.plan(2048, 4096, 8192, out_dtype=torch.bfloat16).tile == 4                # 128 items
    assert tg.plan(1024, 1024, 4096, batch=16).tile == tg.TILE_PINGPONG                # 16 x 16 items
    assert tg.plan(2048, 2048, 8192, out_dtype=torch.bfloat16).tile == 4                # 64 items: 128 x 128
    assert tg.plan(1536, 1536, 8192, out_dtype=torch.bfloat16).tile == 4                # 144 128 x 128 items
    assert tg.plan(1024, 2048, 8192, out_dtype=torch.bfloat16).tile == 11               # 128: the 64 x 64 ring
    assert p.flags & tg.FLAG_PERSIST and p.flags & tg.FLAG_PREFETCH  # MFMA-bound: prefetch during stores
    assert p.workspace_bytes == 0


def test_odd_shapes_take_the_generic_loader():
    st, p = raw_plan(m=17, n=33, k=63)          # K not a multiple of 8
    assert st == tg.TG_OK and p.variant == tg.VARIANT_GENERIC and not p.flags & tg.FLAG_VEC16
    st, p = raw_plan(m=64, n=64, k=64, lda=65)  # odd leading dimension
    assert st == tg.TG_OK and p.variant == tg.VARIANT_GENERIC


def test_lds_budget_matches_the_staging_formula_and_fits():
    for m, n, k in [(256, 256, 256), (1000, 1000, 1000), (8192, 8192, 8192), (2048, 128, 2048), (17, 33, 63),
                    (2048, 2048, 128)]:
        st, p = raw_plan(m=m, n=n, k=k)
        assert st == tg.TG_OK
        if p.variant == tg.VARIANT_TILE and p.tile in (tg.TILE_PINGPONG, tg.TILE_PINGPONG_EPI):
            # three A and two B buffers of one K step
            assert p.lds_bytes == (3 * p.bm * p.bk + 2 * p.bk * p.bn) * 2
        elif p.variant == tg.VARIANT_TILE and p.tile == tg.TILE_PANEL:
            # two B buffers holding all of K
            assert p.lds_bytes == 2 * p.bk * p.bn * 2
        elif p.variant == tg.VARIANT_TILE and p.tile == tg.TILE_KSLICE:
            # a ring of its own for each of the four waves
            assert p.lds_bytes == 4 * roofline.lds_budget(p.bm, p.bn, p.bk, p.stages)
        elif p.variant != tg.VARIANT_SKINNY:
            assert p.lds_bytes == roofline.lds_budget(p.bm, p.bn, p.bk, p.stages)
        assert p.lds_bytes <= roofline.MI355X_LDS_PER_WORKGROUP


def test_run_time_checks_that_need_no_gpu():
    st, p = raw_plan(m=64, n=64, k=64)
    assert st == tg.TG_OK
    L = tg.lib()
    # a stale or foreign plan
    q = tg.GemmPlan.from_buffer_copy(p)
    q.abi_version = 12345
    assert L.gemm_run(ctypes.byref(q), 16, 16, 16, None) == tg.TG_ERR_INVALID
    # null output / inputs with nonzero extents
    assert L.gemm_run(ctypes.byref(p), 16, 16, None, None) == tg.TG_ERR_INVALID
    assert L.gemm_run(ctypes.byref(p), None, 16, 16, None) == tg.TG_ERR_INVALID
    # bad batch arguments; overlapping outputs across the batch
    assert L.bmm_run(ctypes.byref(p), -1, 0, 0, 0, 16, 16, 16, None) == tg.TG_ERR_INVALID
    assert L.bmm_run(ctypes.byref(p), 2, -1, 0, 4096, 16, 16, 16, None) == tg.TG_ERR_INVALID
    assert L.bmm_run(ctypes.byref(p), 2, 0, 0, 64, 16, 16, 16, None) == tg.TG_ERR_INVALID
    # overridden (variant, tile) pairs that do not exist or do not fit
    for variant, tile in [(7, 0), (tg.VARIANT_TILE, 99), (tg.VARIANT_GENERIC, -1), (tg.VARIANT_SKINNY, 0)]:
        q = tg.GemmPlan.from_buffer_copy(p)
        q.variant, q.tile = variant, tile
        assert L.gemm_run(ctypes.byref(q), 16, 16, 16, None) == tg.TG_ERR_UNSUPPORTED
    st, r = raw_plan(m=17, n=33, k=63)
    r.variant = tg.VARIANT_TILE                 # vector loader on a shape it cannot serve
    assert L.gemm_run(ctypes.byref(r), 16, 16, 16, None) == tg.TG_ERR_UNSUPPORTED
    # empty problems launch nothing and succeed
    st, e = raw_plan(m=0, n=64, k=64)
    assert L.gemm_run(ctypes.byref(e), None, None, None, None) == tg.TG_OK
    st, e = raw_plan(m=64, n=64, k=64)
    assert L.bmm_run(ctypes.byref(e), 0, 0, 0, 0, None, None, None, None) == tg.TG_OK


def group_call(problems, tile=-1, count=None, **kw):
    a = dict(in_type=tg.TG_BF16, out_type=tg.TG_FP32, ta=0, tb=0)
    a.update(kw)
    arr = (tg.GroupProblem * max(len(problems), 1))(*[tg.GroupProblem(*q) for q in problems])
    return tg.lib().gemm_group_run(a["in_type"], a["out_type"], a["ta"], a["tb"], arr if problems else None,
                                   len(problems) if count is None else count, tile, None)


GOOD = (64, 64, 64, 64, 64, 64, 4096, 4096, 4096)


def test_group_tile_count():
    assert tg.group_tiles() == 7


@pytest.mark.parametrize("problems,kw,status", [
    ([], dict(), tg.TG_OK),                                            # nothing to do
    ([(0, 64, 64, 64, 64, 64, None, None, None)], dict(), tg.TG_OK),  # empty problems launch nothing
    ([(64, 0, 64, 64, 64, 64, None, None, None)], dict(), tg.TG_OK),
    ([GOOD], dict(count=-1), tg.TG_ERR_INVALID),
    ([GOOD, (64, 64, 64, 32, 64, 64, 4096, 4096, 4096)], dict(), tg.TG_ERR_INVALID),  # lda < k
    ([GOOD, (64, 64, 64, 64, 64, 64, 4096, 4096, None)], dict(), tg.TG_ERR_INVALID),  # null C
    ([GOOD, (64, 64, 64, 64, 64, 64, None, 4096, 4096)], dict(), tg.TG_ERR_INVALID),  # null A, k > 0
    ([(-1, 64, 64, 64, 64, 64, 4096, 4096, 4096)], dict(), tg.TG_ERR_INVALID),
    ([GOOD], dict(tb=2), tg.TG_ERR_INVALID),
    ([GOOD], dict(tile=7), tg.TG_ERR_UNSUPPORTED),
    ([GOOD], dict(tile=-2), tg.TG_ERR_UNSUPPORTED),
    ([GOOD], dict(in_type=tg.TG_FP16, out_type=tg.TG_BF16), tg.TG_ERR_UNSUPPORTED),
])
def test_group_argument_checks(problems, kw, status):
    """Every problem is validated before anything is enqueued (no device call here)."""
    count = kw.pop("count", None)
    tile = kw.pop("tile", -1)
    assert group_call(problems, tile=tile, count=count, **kw) == status


def test_group_null_array_with_count():
    assert tg.lib().gemm_group_run(tg.TG_BF16, tg.TG_FP32, 0, 0, None, 3, -1, None) == tg.TG_ERR_INVALID


def attn_call(**kw):
    """attention_fwd with a valid 2 x 256 x 256 x 128 bf16 problem, overridden by kw."""
    a = dict(in_type=tg.TG_BF16, out_type=tg.TG_FP32, batch=2, n_q=256, n_k=256, head_dim=128, scale=0.125,
             Q=4096, ldq=128, sq=256 * 128, K=4096, ldk=128, sk=256 * 128, V=4096, ldv=128, sv=256 * 128,
             O=4096, ldo=128, so=256 * 128)
    a.update(kw)
    return tg.lib().attention_fwd(a["in_type"], a["out_type"], a["batch"], a["n_q"], a["n_k"], a["head_dim"],
                                  ctypes.c_float(a["scale"]), a["Q"], a["ldq"], a["sq"], a["K"], a["ldk"], a["sk"],
                                  a["V"], a["ldv"], a["sv"], a["O"], a["ldo"], a["so"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), tg.TG_ERR_INVALID),
    (dict(n_q=-1), tg.TG_ERR_INVALID),
    (dict(n_k=0), tg.TG_ERR_INVALID),                  # softmax over no keys
    (dict(scale=0.0), tg.TG_ERR_INVALID),
    (dict(scale=-0.5), tg.TG_ERR_INVALID),
    (dict(scale=float("inf")), tg.TG_ERR_INVALID),
    (dict(scale=float("nan")), tg.TG_ERR_INVALID),
    (dict(ldq=127), tg.TG_ERR_INVALID),
    (dict(ldo=64), tg.TG_ERR_INVALID),
    (dict(sk=-1), tg.TG_ERR_INVALID),
    (dict(so=128), tg.TG_ERR_INVALID),                 # heads' outputs overlap
    (dict(O=None), tg.TG_ERR_INVALID),
    (dict(K=None), tg.TG_ERR_INVALID),
    (dict(in_type=tg.TG_FP32), tg.TG_ERR_UNSUPPORTED),
    (dict(in_type=tg.TG_FP16, out_type=tg.TG_BF16), tg.TG_ERR_UNSUPPORTED),
    (dict(head_dim=96, ldq=128, ldk=128, ldv=128, ldo=128), tg.TG_ERR_UNSUPPORTED),
    (dict(ldk=132), tg.TG_ERR_UNSUPPORTED),            # not a multiple of 8
    (dict(V=4096 + 2), tg.TG_ERR_UNSUPPORTED),         # misaligned base
    (dict(ldq=1 << 20, sq=256 << 20), tg.TG_ERR_UNSUPPORTED),
    (dict(n_k=1 << 23, sk=128 << 23, sv=128 << 23), tg.TG_ERR_UNSUPPORTED),   # a head's K spans 2 GiB
    (dict(n_k=1 << 22, ldv=512, sv=512 << 22), tg.TG_ERR_UNSUPPORTED),       # a head's V spans 2 GiB
    (dict(batch=0, Q=None, K=None, V=None, O=None), tg.TG_OK),   # nothing to do
    (dict(n_q=0, n_k=0, O=None), tg.TG_OK),
])
def test_attention_argument_checks(kw, status):
    """Every rejection (and the empty launches) happens before any device call."""
    assert attn_call(**kw) == status


def test_page_figures_pin_the_roofline_arithmetic():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))
    r = g["ridge_a100_fp16"]
    assert roofline.ridge(r["peak_flops"], r["peak_bytes"]) == r["ridge"]
    f = g["gemm_fp16_bytes_formula"]
    assert roofline.gemm_flops(f["m"], f["n"], f["k"]) == f["flops"]
    assert roofline.gemm_bytes(f["m"], f["n"], f["k"], in_size=2, out_size=2) == f["bytes"]
    s = g["smem_overflow_example"]
    assert roofline.lds_budget(s["bm"], s["bn"], s["bk"], s["stages"], s["elem"]) == s["bytes"] > s["a100_limit_bytes"]
    a = g["accumulator_example"]
    assert roofline.accumulator_bytes(a["bm"], a["bn"]) == a["bytes"]
    # the same arithmetic on MI355X: the 8192^3 GEMM is MFMA-bound, the M=16 one HBM-bound
    assert roofline.bound(8192, 8192, 8192, out_size=2) == "mfma"
    assert roofline.bound(16, 8192, 8192, out_size=2) == "hbm"


def test_python_constants_match_the_header():
    """The binding's copies of the header's tile and flag numbers."""
    import re
    text = open(tg.HEADER).read()
    defs = dict(re.findall(r"#define\s+(TG_\w+)\s+(0x[0-9a-fA-F]+|\d+)", text))
    assert int(defs["TG_TILE_PINGPONG"], 0) == tg.TILE_PINGPONG
    assert int(defs["TG_TILE_PINGPONG_EPI"], 0) == tg.TILE_PINGPONG_EPI
    assert int(defs["TG_TILE_PANEL"], 0) == tg.TILE_PANEL
    assert int(defs["TG_TILE_KSLICE"], 0) == tg.TILE_KSLICE
    assert int(defs["TG_SPLITK_MAX"], 0) == tg.SPLITK_MAX
    m = re.search(r"#define\s+TG_SPLITK_SCRATCH_BYTES\s+\((\d+)ull << (\d+)\)", text)
    assert int(m.group(1)) << int(m.group(2)) == tg.SPLITK_SCRATCH_BYTES
    for name in ("EVEN_K", "VEC16", "ROTATE_K", "PERSIST", "PREFETCH", "STREAM_C"):
        assert int(defs["TG_FLAG_" + name], 0) == getattr(tg, "FLAG_" + name)


def test_splitk_host_side():
    """Workspace size, split suggestion and argument checks of gemm_splitk_run
    (all answered on the host, before anything is enqueued)."""
    import torch
    L = tg.lib()
    p = tg.plan(1024, 1000, 65536, out_dtype=torch.bfloat16)
    # ks = ceil(65536 / 8) = 8192 -> 8 parts of 1024 rows x ldw = 1000 rounded up to 8 floats
    assert tg.splitk_workspace_bytes(p, 8) == 8 * 1024 * 1000 * 4
    # K = 1000 in 3 parts: ks = 336 (a multiple of 8) -> parts of 336, 336, 328
    q = tg.plan(64, 36, 1000)
    assert tg.splitk_workspace_bytes(q, 3) == 3 * 64 * 40 * 4
    # more splits than 8-element parts: K = 24 in 8 splits -> ks = 8, 3 parts
    r = tg.plan(16, 16, 24)
    assert tg.splitk_workspace_bytes(r, 8) == 3 * 16 * 16 * 4
    assert tg.splitk_workspace_bytes(tg.plan(16, 16, 0), 4) == 0
    for bad in (0, -1, tg.SPLITK_MAX + 1):
        assert tg.splitk_workspace_bytes(p, bad) == 0
    # suggestion: 16 tiles of 256 x 256 and a long K -> 16 parts (one item per CU); many tiles or short K -> 1
    assert tg.splitk_choose(p) == 16
    assert tg.splitk_choose(tg.plan(1024, 1024, 1024)) == 1
    assert tg.splitk_choose(tg.plan(4096, 4096, 65536)) == 1
    assert tg.splitk_choose(tg.plan(2048, 2048, 65536)) == 4  # 64 tiles of 256 x 256
    assert tg.splitk_choose(tg.plan(1536, 1536, 8192)) == 4   # 36 tiles: 144 items of 2048-deep parts
    assert tg.splitk_choose(tg.plan(2048, 2048, 4096)) == 1   # only 128 items of 2048-deep parts
    assert tg.splitk_choose(tg.plan(1024, 2048, 8192)) == 1
    assert tg.splitk_choose(tg.plan(128, 128, 4096)) == 8  # K / 512
    assert tg.splitk_choose(tg.plan(128, 128, 1 << 20)) == tg.SPLITK_MAX
    stale = tg.GemmPlan.from_buffer_copy(p)
    stale.abi_version = 0
    assert tg.splitk_choose(stale) == 1 and tg.splitk_workspace_bytes(stale, 2) == 0
    A = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its checks first
    need = tg.splitk_workspace_bytes(p, 8)
    ws = ctypes.c_void_p(1 << 24)
    calls = [
        (stale, 8, ws, need, A, A, A),          # stale plan
        (p, 0, ws, need, A, A, A),              # splits out of range
        (p, tg.SPLITK_MAX + 1, ws, need, A, A, A),
        (p, 8, ws, need - 1, A, A, A),          # workspace too small
        (p, 8, None, need, A, A, A),            # no workspace
        (p, 8, ctypes.c_void_p((1 << 24) + 4), need, A, A, A),  # misaligned workspace
        (p, 8, ws, need, None, A, A),           # null A with K > 0
        (p, 8, ws, need, A, A, None),           # null C
    ]
    for pl, s, w, nb, a, b, c in calls:
        assert L.gemm_splitk_run(ctypes.byref(pl), s, w, nb, a, b, c, None) == tg.TG_ERR_INVALID
    assert L.gemm_splitk_run(None, 8, ws, need, A, A, A, None) == tg.TG_ERR_INVALID
    # an empty product enqueues nothing
    e = tg.plan(0, 16, 64)
    assert L.gemm_splitk_run(ctypes.byref(e), 2, None, 0, None, None, None, None) == tg.TG_OK
    # the no-allocation variant: the same argument checks, and sizes beyond its
    # fixed array refused before any device call
    for pl, s, w, nb, a, b, c in calls:
        if w is ws and nb == need:
            assert L.gemm_splitk_run_noalloc(ctypes.byref(pl), s, a, b, c, None) == tg.TG_ERR_INVALID
    big = tg.plan(1024, 1032, 65536)
    assert tg.splitk_workspace_bytes(big, 16) > tg.SPLITK_SCRATCH_BYTES
    assert L.gemm_splitk_run_noalloc(ctypes.byref(big), 16, A, A, A, None) == tg.TG_ERR_TOO_LARGE
    assert L.gemm_splitk_run_noalloc(ctypes.byref(e), 2, None, None, None, None) == tg.TG_OK


# ---- the Python binding's operand checks (CPU tensors: the structural checks
# run before the device check, so each bad layout is refused by its own message
# and nothing reaches the library)

def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("make,msg", [
    (lambda: _bf(4, 8, 2), "must be a 2-D"),                              # 3-D where a matrix is expected
    (lambda: _bf(8).expand(4, 8), "rows overlap"),                        # row stride 0
    (lambda: _bf(8, 4).t(), "contiguous last dimension"),                 # transposed view
    (lambda: _bf(4, 16)[:, ::2], "contiguous last dimension"),            # strided columns
    (lambda: _bf(4, 8), "GPU tensor"),                                    # well-formed, but on the host
])
def test_binding_rejects_bad_operand_layouts(make, msg):
    with pytest.raises(ValueError, match=msg):
        tg.gemm(make(), _bf(8, 8))


def test_binding_rejects_bad_outputs_before_launch():
    import torch
    A, B = _bf(4, 8), _bf(8, 6)
    with pytest.raises(ValueError, match="wrong shape or dtype"):
        tg._check_out(_bf(4, 6), (4, 6), torch.float32)             # bf16 out, fp32 requested
    with pytest.raises(ValueError, match="contiguous last dimension"):
        tg._check_out(torch.zeros(6, 4).t(), (4, 6), torch.float32)  # transposed out
    with pytest.raises(ValueError, match="rows overlap"):
        tg._check_out(torch.zeros(6).expand(4, 6), (4, 6), torch.float32)
    with pytest.raises(ValueError, match="batch overlap"):
        tg._check_out(torch.zeros(4, 6).expand(3, 4, 6), (3, 4, 6), torch.float32, (3,))
    with pytest.raises(ValueError, match="must be a 3-D"):
        tg.bmm(A, B)
    with pytest.raises(ValueError, match="must be a 2-D"):
        tg.gemm_splitk(_bf(2, 4, 8), B)
    with pytest.raises(ValueError, match="must be a 2-D"):
        tg.gemm_group([_bf(2, 4, 8)], [B])
    # a well-formed host output still stops at the device check
    with pytest.raises(ValueError, match="GPU tensor"):
        tg._check_out(torch.zeros(3, 4, 6), (3, 4, 6), torch.float32, (3,))
