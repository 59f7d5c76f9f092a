"""Parity of the fused attention forward pass (attention_fwd) with the oracle.

Tolerance, derived from the kernel's arithmetic (per output element (r, c)):
  * the probabilities enter the product with V rounded to the input type:
    relative error <= u_p = 2^-8 (bf16) or 2^-11 (fp16), so the weighted sum
    moves by at most u_p * (P|V|)[r, c], where P|V| is the attention applied
    to |V| (the oracle computes it exactly);
  * fp32 scores: each is a d-term fp32 sum of exact products, error
    <= d * 2^-24 * sum|q k|, which scales p by at most
    e_s = ln2 * c * d^2 * 2^-24 * max|Q| * max|K| (c = scale * log2 e);
  * fp32 sums over n_k keys (numerator and row sum), the exp2 instruction
    and the final division: e_a = n_k * 2^-24 + 2^-21 each;
  * fp16 probabilities below 2^-14 are subnormal: absolute error 2^-25 each.
    |O - Oref| <= (u_p + 2 (e_s + e_a)) (P|V|) + [fp16] n_k 2^-25 max|V|
plus half an output ulp for a 16-bit output (parity.bound).

A second family has probabilities that are exact powers of two (integer
scores, scale = ln 2, so 2^(s - max) exactly), where every sum is exact in
fp32 and only the final division rounds: there the kernel must agree with the
oracle to a few fp32 ulps, which a dropped, doubled or misplaced key would
break by orders of magnitude.
"""
import math

import numpy as np
import pytest
import torch

import matmul_tiled_bf16_amd as tg
import oracle
import synth
from parity import bound, to_gpu, torch_out_dtype, values

pytestmark = pytest.mark.gpu

U_P = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
TIN = {"bf16": torch.bfloat16, "fp16": torch.float16}
CANARY = -12345.0


def attn_tolerance(Q, K, V, pv_abs, n_k, d, scale, in_dtype):
    mq, mk, mv = (oracle.max_abs(X, in_dtype) for X in (Q, K, V))
    c = scale * math.log2(math.e)
    e_s = math.log(2) * c * d * d * 2.0 ** -24 * mq * mk
    e_a = n_k * 2.0 ** -24 + 2.0 ** -21
    t = (U_P[in_dtype] + 2 * (e_s + e_a)) * pv_abs
    if in_dtype == "fp16":
        t = t + n_k * 2.0 ** -25 * mv
    return t


def make_inputs(rng, batch, n_q, n_k, d, in_dtype, pad=0):
    """Q, K, V ~ N(0,1) with leading dimension d + pad (padding NaN)."""
    nan = np.uint16(0x7FC0 if in_dtype == "bf16" else 0x7E00)
    out = []
    for rows in (n_q, n_k, n_k):
        X = np.full((batch, rows, d + pad), nan, dtype=np.uint16)
        X[:, :, :d] = synth.draw(rng, (batch, rows, d), "normal", 1.0, dtype=in_dtype)
        out.append(X)
    return out


def run(Q, K, V, batch, n_q, n_k, d, scale, in_dtype, out_dtype, ldo=None):
    """Launch through the C ABI; returns O as float64 [batch, n_q, ldo] (canaries in the padding)."""
    ld = Q.shape[-1]
    ldo = ldo or d
    Qg, Kg, Vg = (to_gpu(X, in_dtype) for X in (Q, K, V))
    O = torch.full((batch, n_q, ldo), CANARY, dtype=torch_out_dtype(out_dtype), device="cuda")
    tg.attention_fwd(tg._dtype_code(TIN[in_dtype]), tg._dtype_code(torch_out_dtype(out_dtype)), batch, n_q, n_k, d,
                     scale, Qg, ld, n_q * ld, Kg, K.shape[-1], n_k * K.shape[-1], Vg, V.shape[-1], n_k * V.shape[-1],
                     O, ldo, n_q * ldo)
    torch.cuda.synchronize()
    return values(O)


def reference(Q, K, V, batch, n_q, n_k, d, scale, in_dtype, rows=None):
    ld = Q.shape[-1]
    kw = dict(n_q=n_q, n_k=n_k, head_dim=d, scale=scale, batch=batch, ldq=ld, ldk=K.shape[-1], ldv=V.shape[-1],
              in_dtype=in_dtype, rows=rows)
    o = oracle.attention(Q, K, V, **kw)
    pv = oracle.attention(Q, K, V & np.uint16(0x7FFF), **kw)
    return o, pv


CASES = [  # batch, n_q, n_k, d
    (2, 200, 300, 128),   # ragged query and key blocks
    (3, 128, 64, 64),     # exactly one block of each
    (1, 1, 1, 128),       # one query, one key: O = V
    (2, 257, 129, 64),    # one past a block boundary on both sides
    (1, 130, 1000, 128),  # many key blocks, ragged last
    (1, 64, 2, 128),      # fewer keys than a lane half holds
]


@pytest.mark.parametrize("in_dtype,out_dtype", [("bf16", "fp32"), ("bf16", "bf16"), ("fp16", "fp32"),
                                                ("fp16", "fp16")])
@pytest.mark.parametrize("case", CASES)
def test_attention_matches_oracle(case, in_dtype, out_dtype):
    batch, n_q, n_k, d = case
    rng = np.random.default_rng(sum(case) * 7 + len(in_dtype + out_dtype))
    Q, K, V = make_inputs(rng, batch, n_q, n_k, d, in_dtype)
    scale = 1.0 / math.sqrt(d)
    print(f"attention {case} {in_dtype}->{out_dtype}", flush=True)
    o = run(Q, K, V, batch, n_q, n_k, d, scale, in_dtype, out_dtype)
    oref, pv = reference(Q, K, V, batch, n_q, n_k, d, scale, in_dtype)
    t = attn_tolerance(Q, K, V, pv, n_k, d, scale, in_dtype)
    err = np.abs(o - oref)
    b = bound(oref, t, out_dtype)
    assert np.all(np.isfinite(o))
    bad = err > b
    assert not bad.any(), (f"{int(bad.sum())} over tolerance, worst ratio {float(np.max(err / b)):.3g} at "
                           f"{np.unravel_index(np.argmax(err / b), err.shape)}")


@pytest.mark.parametrize("in_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("n_k", [1, 37, 64, 100, 191])
def test_attention_exact_probabilities(n_k, in_dtype):
    """Integer scores in [-3, 3] and scale = ln 2: every p is a power of two
    >= 2^-6 and every sum is exact in fp32 (integer V), so only the division
    by the row sum rounds."""
    batch, n_q, d = 2, 160, 128
    rng = np.random.default_rng(1000 + n_k)
    scale = float(np.float32(math.log(2.0)))
    Qv = np.zeros((batch, n_q, d))
    Kv = np.zeros((batch, n_k, d))
    cols = rng.choice(d, size=3, replace=False)
    Qv[:, :, cols] = rng.integers(-1, 2, size=(batch, n_q, 3))
    Kv[:, :, cols] = rng.integers(-1, 2, size=(batch, n_k, 3))
    Vv = rng.integers(-4, 5, size=(batch, n_k, d)).astype(np.float64)
    enc = lambda X: oracle.round_to(X, in_dtype)  # exact: small integers
    Q, K, V = enc(Qv), enc(Kv), enc(Vv)
    o = run(Q, K, V, batch, n_q, n_k, d, scale, in_dtype, "fp32")
    oref, pv = reference(Q, K, V, batch, n_q, n_k, d, scale, in_dtype)
    # the division rounds twice (reciprocal, product); the oracle's exp(s*scale)
    # differs from 2^s by |s|*2e-9 relative
    t = 2.0 ** -21 * pv + 2.0 ** -21 * np.abs(oref)
    err = np.abs(o - oref)
    assert np.all(err <= t), f"worst {float(np.max(err - t)):.3g} over, max err {float(err.max()):.3g}"


def test_attention_padded_rows_and_canaries():
    """Leading dimensions with NaN padding (never read into the result) and an
    output with padded rows (the padding keeps its canaries)."""
    batch, n_q, n_k, d = 3, 150, 200, 64
    rng = np.random.default_rng(77)
    Q, K, V = make_inputs(rng, batch, n_q, n_k, d, "bf16", pad=24)
    scale = 0.1
    o = run(Q, K, V, batch, n_q, n_k, d, scale, "bf16", "fp32", ldo=d + 16)
    assert np.all(o[:, :, d:] == CANARY)
    oref, pv = reference(Q, K, V, batch, n_q, n_k, d, scale, "bf16")
    t = attn_tolerance(Q, K, V, pv, n_k, d, scale, "bf16")
    assert np.all(np.abs(o[:, :, :d] - oref) <= t)


def test_attention_full_size_sampled():
    """The benchmark's workload (128 heads, 2048 x 2048, d = 128, fp32 out) in
    its launch configuration, checked on seeded sampled rows plus block edges."""
    p = synth.attention_fwd()
    rows = synth.attention_rows(5, p.batch, p.n_q)
    Qg, Kg, Vg = (to_gpu(X) for X in (p.Q, p.K, p.V))
    O = tg.attention(Qg, Kg, Vg, scale=p.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = values(O[torch.from_numpy(rows[:, 0]).cuda(), torch.from_numpy(rows[:, 1]).cuda()])
    kw = dict(n_q=p.n_q, n_k=p.n_k, head_dim=p.d, scale=p.scale, batch=p.batch, rows=rows)
    oref = oracle.attention(p.Q, p.K, p.V, **kw)
    pv = oracle.attention(p.Q, p.K, p.V & np.uint16(0x7FFF), **kw)
    t = attn_tolerance(p.Q, p.K, p.V, pv, p.n_k, p.d, p.scale, "bf16")
    err = np.abs(got - oref)
    assert np.all(err <= t), f"worst ratio {float(np.max(err / t)):.3g}"
    # the typical error sits far below the worst-case bound
    assert float(np.median(err / t)) < 0.1


def test_attention_deterministic():
    p = synth.attention_fwd(seed=9, batch=4, seq=512, head=128)
    Qg, Kg, Vg = (to_gpu(X) for X in (p.Q, p.K, p.V))
    a = tg.attention(Qg, Kg, Vg, scale=p.scale)
    b = tg.attention(Qg, Kg, Vg, scale=p.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
