"""Pins for the CPU oracle, checked against things other than itself.

Each test fixes a property that the definition C = op(A) op(B) or the 16-bit
formats determine independently of the oracle's code: hand-worked products,
exact identities (identity and permutation factors, explicit transposes),
integer inputs against numpy's int64 matmul, exact rational sums on tiny
shapes, closed forms, and every bf16/fp16 bit pattern against torch/numpy
conversions.  A dropped term, a flipped sign, a swapped index or a transposed
operand in the oracle fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x) -> np.ndarray:
    """Exact encoding of values that are representable in bf16 (torch's conversion)."""
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    back = t.to(torch.bfloat16)
    assert torch.equal(back.float(), t), "value not representable in bf16"
    return back.view(torch.int16).numpy().view(np.uint16)


def fp16_bits(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    h = a.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), a)
    return h.view(np.uint16)


def stored(X: np.ndarray, trans: int) -> np.ndarray:
    """The array a caller stores so that op(stored) == X."""
    return np.ascontiguousarray(X.T) if trans else np.ascontiguousarray(X)


def rand_bf16(rng, shape, scale=1.0):
    return synth.draw(rng, shape, "normal", scale)


# ---------------------------------------------------------------- codecs ---

def test_decode_every_bf16_pattern_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_every_fp16_pattern_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    u[::3] = (u[::3] & 0xFFFF0000) | 0x8000       # exact ties
    u[1::7] = (u[1::7] & 0xFFFF0000) | 0x7FFF
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.round_to(x.astype(np.float64), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_round_fp16_matches_numpy_on_doubles():
    rng = np.random.default_rng(8)
    x = np.concatenate([
        rng.standard_normal(200_000) * 1000.0,
        rng.standard_normal(100_000) * 1e-5,              # subnormal range
        (rng.integers(-4096, 4096, 50_000) + 0.5) * 2.0 ** -10,  # ties
        np.array([65504.0, 65519.99, 65520.0, 1e6, -1e6, 0.0, -0.0]),
    ])
    got = oracle.round_to(x, "fp16")
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_round_hand_cases(fmt):
    cases = json.load(open(os.path.join(GOLD, "hand_examples.json")))[f"{fmt}_rounding"]
    x = np.array([c["x"] for c in cases])
    want = np.array([int(c["bits"], 16) for c in cases], dtype=np.uint16)
    assert np.array_equal(oracle.round_to(x, fmt), want), [c["why"] for c in cases]


# ------------------------------------------------------- hand examples ---

@pytest.mark.parametrize("ta", [0, 1])
@pytest.mark.parametrize("tb", [0, 1])
def test_hand_worked_products(ta, tb):
    for p in json.load(open(os.path.join(GOLD, "hand_examples.json")))["products"]:
        A = np.array(p["A"], dtype=np.float64)
        B = np.array(p["B"], dtype=np.float64)
        C = np.array(p["C"], dtype=np.float64)
        m, k = A.shape
        n = B.shape[1]
        got = oracle.gemm(bf16_bits(stored(A, ta)), bf16_bits(stored(B, tb)), m=m, n=n, k=k,
                          trans_a=ta, trans_b=tb)[0]
        assert np.array_equal(got, C), p["name"]


# ------------------------------------------------------------ identities ---

@pytest.mark.parametrize("ta", [0, 1])
@pytest.mark.parametrize("tb", [0, 1])
def test_identity_factor_returns_other_operand(ta, tb):
    rng = np.random.default_rng(11)
    m, k = 37, 53
    X = rand_bf16(rng, (m, k))
    Xv = oracle.decode(X)
    I = bf16_bits(np.eye(k))
    got = oracle.gemm(stored(X, ta), I, m=m, n=k, k=k, trans_a=ta, trans_b=tb)[0]
    assert np.array_equal(got, Xv)
    # identity on the left
    I2 = bf16_bits(np.eye(m))
    Y = rand_bf16(rng, (m, k))
    got = oracle.gemm(I2, stored(Y, tb), m=m, n=k, k=m, trans_a=ta, trans_b=tb)[0]
    assert np.array_equal(got, oracle.decode(Y))


@pytest.mark.parametrize("ta", [0, 1])
@pytest.mark.parametrize("tb", [0, 1])
def test_permutation_factors_permute_exactly(ta, tb):
    rng = np.random.default_rng(12)
    m, k, n = 19, 23, 29
    X = rand_bf16(rng, (k, n))
    perm = rng.permutation(m) % k
    P = np.zeros((m, k))
    P[np.arange(m), perm] = 1.0  # row i of P picks row perm[i] of X
    got = oracle.gemm(bf16_bits(stored(P, ta)), stored(X, tb), m=m, n=n, k=k, trans_a=ta, trans_b=tb)[0]
    assert np.array_equal(got, oracle.decode(X)[perm, :])
    Y = rand_bf16(rng, (m, k))
    colperm = rng.permutation(n) % k
    Q = np.zeros((k, n))
    Q[colperm, np.arange(n)] = 1.0  # column j of Q picks column colperm[j] of Y
    got = oracle.gemm(stored(Y, ta), bf16_bits(stored(Q, tb)), m=m, n=n, k=k, trans_a=ta, trans_b=tb)[0]
    assert np.array_equal(got, oracle.decode(Y)[:, colperm])


def test_explicit_transpose_is_bitwise_equivalent():
    rng = np.random.default_rng(13)
    m, n, k = 41, 35, 67
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (k, n))
    ref = oracle.gemm(A, B, m=m, n=n, k=k)
    for ta in (0, 1):
        for tb in (0, 1):
            got = oracle.gemm(stored(A, ta), stored(B, tb), m=m, n=n, k=k, trans_a=ta, trans_b=tb)
            assert np.array_equal(got, ref), (ta, tb)


# ------------------------------------------------------ integer inputs ---

@pytest.mark.parametrize("in_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ta", [0, 1])
@pytest.mark.parametrize("tb", [0, 1])
def test_integer_inputs_equal_int64_matmul(in_dtype, ta, tb):
    rng = np.random.default_rng(14 + 2 * ta + tb)
    batch, m, n, k = 3, 33, 47, 130
    Ai = rng.integers(-8, 9, size=(batch, m, k))
    Bi = rng.integers(-8, 9, size=(batch, k, n))
    enc = bf16_bits if in_dtype == "bf16" else fp16_bits
    As = np.stack([stored(Ai[b], ta) for b in range(batch)])
    Bs = np.stack([stored(Bi[b], tb) for b in range(batch)])
    got = oracle.gemm(enc(As), enc(Bs), m=m, n=n, k=k, trans_a=ta, trans_b=tb, batch=batch,
                      stride_a=m * k, stride_b=k * n, in_dtype=in_dtype)
    ref = np.matmul(Ai.astype(np.int64), Bi.astype(np.int64))
    assert np.array_equal(got, ref.astype(np.float64))


# ------------------------------------------------ brute force, tiny sizes ---

def test_tiny_shapes_match_exact_rational_sums():
    rng = np.random.default_rng(15)
    u = 2.0 ** -53
    for trial in range(60):
        m, n, k = (int(v) for v in rng.integers(1, 6, size=3))
        ta, tb = (int(v) for v in rng.integers(0, 2, size=2))
        A = rand_bf16(rng, (m, k), 3.0)
        B = rand_bf16(rng, (k, n), 3.0)
        Ad, Bd = oracle.decode(A), oracle.decode(B)
        got = oracle.gemm(stored(A, ta), stored(B, tb), m=m, n=n, k=k, trans_a=ta, trans_b=tb)[0]
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(Ad[i, kk]) * Fraction(Bd[kk, j]) for kk in range(k))
                bound = k * u * sum(abs(Ad[i, kk] * Bd[kk, j]) for kk in range(k))
                assert abs(Fraction(got[i, j]) - exact) <= Fraction(bound), (trial, i, j)
        np_ref = Ad @ Bd
        bound = k * u * (np.abs(Ad) @ np.abs(Bd)) * 2
        assert np.all(np.abs(got - np_ref) <= bound)


# --------------------------------------------------------- closed forms ---

def test_ones_give_k_and_scaling_is_exact():
    m, n, k = 20, 30, 777
    ones_a = bf16_bits(np.ones((m, k)))
    ones_b = bf16_bits(np.ones((k, n)))
    assert np.array_equal(oracle.gemm(ones_a, ones_b, m=m, n=n, k=k)[0], np.full((m, n), float(k)))
    rng = np.random.default_rng(16)
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (k, n))
    A2 = bf16_bits(2.0 * oracle.decode(A))
    c1 = oracle.gemm(A, B, m=m, n=n, k=k)
    c2 = oracle.gemm(A2, B, m=m, n=n, k=k)
    assert np.array_equal(c2, 2.0 * c1)
    Bneg = bf16_bits(-oracle.decode(B))
    assert np.array_equal(oracle.gemm(A, Bneg, m=m, n=n, k=k), -c1)


def test_empty_k_gives_zeros_and_empty_mn_gives_empty():
    z = np.zeros(0, dtype=np.uint16)
    out = oracle.gemm(z, z, m=5, n=7, k=0, lda=1, ldb=7)
    assert out.shape == (1, 5, 7) and np.all(out == 0.0)
    out = oracle.gemm(z, np.zeros(21, np.uint16), m=0, n=7, k=3)
    assert out.shape == (1, 0, 7)


# ------------------------------------------------- addressing features ---

def test_batch_strides_and_broadcast():
    rng = np.random.default_rng(17)
    batch, m, n, k = 4, 9, 11, 13
    A = rand_bf16(rng, (batch, m, k))
    B = rand_bf16(rng, (batch, k, n))
    full = oracle.gemm(A, B, m=m, n=n, k=k, batch=batch, stride_a=m * k, stride_b=k * n)
    for b in range(batch):
        assert np.array_equal(full[b], oracle.gemm(A[b], B[b], m=m, n=n, k=k)[0])
    bc = oracle.gemm(A, B[0], m=m, n=n, k=k, batch=batch, stride_a=m * k, stride_b=0)
    for b in range(batch):
        assert np.array_equal(bc[b], oracle.gemm(A[b], B[0], m=m, n=n, k=k)[0])


def test_leading_dimension_padding_is_never_read():
    rng = np.random.default_rng(18)
    m, n, k = 17, 19, 23
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (k, n))
    ref = oracle.gemm(A, B, m=m, n=n, k=k)
    nan = np.uint16(0x7FC0)
    Ap = np.full((m, k + 5), nan, dtype=np.uint16)
    Ap[:, :k] = A
    Bp = np.full((k, n + 3), nan, dtype=np.uint16)
    Bp[:, :n] = B
    got = oracle.gemm(Ap, Bp, m=m, n=n, k=k, lda=k + 5, ldb=n + 3)
    assert np.array_equal(got, ref)


def test_sampled_elements_equal_full_result():
    rng = np.random.default_rng(19)
    batch, m, n, k = 3, 50, 60, 70
    A = rand_bf16(rng, (batch, k, m))
    B = rand_bf16(rng, (batch, n, k))
    kw = dict(m=m, n=n, k=k, trans_a=1, trans_b=1, batch=batch, stride_a=m * k, stride_b=k * n)
    full = oracle.gemm(A, B, **kw)
    idx = synth.sample_indices(5, batch, m, n, count=500)
    got = oracle.gemm(A, B, idx=idx, **kw)
    assert np.array_equal(got, full[idx[:, 0], idx[:, 1], idx[:, 2]])
    with pytest.raises(IndexError):
        oracle.gemm(A, B, idx=np.array([[0, m, 0]]), **kw)


def test_max_abs_matches_decoded_maximum():
    rng = np.random.default_rng(20)
    X = rand_bf16(rng, (300, 301), 5.0)
    assert oracle.max_abs(X) == np.max(np.abs(oracle.decode(X)))


# ----------------------------------------------------------------------------
# fused attention forward: O = softmax(scale * Q K^T) V (no mask)
# ----------------------------------------------------------------------------

def _attn_inputs(seed, batch, n_q, n_k, d, dist=("normal", 1.0)):
    rng = np.random.default_rng(seed)
    Q = synth.draw(rng, (batch, n_q, d), *dist)
    K = synth.draw(rng, (batch, n_k, d), *dist)
    V = synth.draw(rng, (batch, n_k, d), *dist)
    return Q, K, V


def test_attention_identical_keys_give_the_mean_of_v():
    """All scores of a row equal -> uniform weights -> O is the plain mean of V's rows."""
    Q, K, V = _attn_inputs(11, 2, 3, 9, 8)
    K[:] = K[:, :1, :]                       # every key is the first key
    o = oracle.attention(Q, K, V, n_q=3, n_k=9, head_dim=8, scale=0.7, batch=2)
    mean = oracle.decode(V).reshape(2, 9, 8).mean(axis=1)
    np.testing.assert_allclose(o, np.broadcast_to(mean[:, None, :], o.shape), rtol=0, atol=1e-15)


def test_attention_single_key_returns_that_value_row():
    Q, K, V = _attn_inputs(12, 2, 4, 1, 16)
    o = oracle.attention(Q, K, V, n_q=4, n_k=1, head_dim=16, scale=3.0, batch=2)
    v = oracle.decode(V).reshape(2, 1, 16)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))


def test_attention_dominant_key_selects_its_value_row():
    """One key aligned with the query and a large scale: weight ~1 on it, < exp(-40) elsewhere."""
    d, n_k = 8, 6
    Q = np.zeros((1, 1, d), np.uint16)
    K = np.zeros((1, n_k, d), np.uint16)
    Q[0, 0, 0] = 0x3F80                      # q = e0 (bf16 1.0)
    for j in range(n_k):
        K[0, j, 0] = 0x3F80 if j == 4 else 0x3F00   # key 4 scores 1.0, the others 0.5
    rng = np.random.default_rng(13)
    V = synth.draw(rng, (1, n_k, d), "normal", 1.0)
    o = oracle.attention(Q, K, V, n_q=1, n_k=n_k, head_dim=d, scale=100.0)
    v = oracle.decode(V).reshape(n_k, d)
    np.testing.assert_allclose(o[0, 0], v[4], rtol=0, atol=6 * np.exp(-50.0) * np.abs(v).max() + 1e-300)


def test_attention_equals_gemm_then_numpy_softmax_then_numpy_matmul():
    """The same definition composed from the pinned GEMM oracle, numpy's softmax
    arithmetic and numpy's matmul."""
    b, n_q, n_k, d = 3, 17, 33, 24
    Q, K, V = _attn_inputs(14, b, n_q, n_k, d)
    scale = 1.0 / np.sqrt(d)
    o = oracle.attention(Q, K, V, n_q=n_q, n_k=n_k, head_dim=d, scale=scale, batch=b)
    s = oracle.gemm(Q, K, m=n_q, n=n_k, k=d, trans_b=1, batch=b, stride_a=n_q * d, stride_b=n_k * d) * scale
    w = np.exp(s - s.max(axis=2, keepdims=True))
    p = w / w.sum(axis=2, keepdims=True)
    ref = p @ oracle.decode(V).reshape(b, n_k, d)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_attention_tiny_brute_force_in_pure_python():
    import math
    n_q, n_k, d = 2, 5, 3
    Q, K, V = _attn_inputs(15, 1, n_q, n_k, d)
    q, k, v = (oracle.decode(x).reshape(-1, d).tolist() for x in (Q, K, V))
    scale = 0.9
    o = oracle.attention(Q, K, V, n_q=n_q, n_k=n_k, head_dim=d, scale=scale)
    for i in range(n_q):
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in range(n_k)]
        w = [math.exp(x) for x in s]        # small scores: no shift needed
        den = math.fsum(w)
        for c in range(d):
            want = math.fsum(w[j] * v[j][c] for j in range(n_k)) / den
            assert abs(o[0, i, c] - want) <= 1e-14 * max(1.0, abs(want))


def test_attention_is_invariant_to_key_order_and_to_a_common_score_shift():
    b, n_q, n_k, d = 2, 5, 12, 8
    Q, K, V = _attn_inputs(16, b, n_q, n_k, d)
    o = oracle.attention(Q, K, V, n_q=n_q, n_k=n_k, head_dim=d, scale=0.5, batch=b)
    perm = np.random.default_rng(17).permutation(n_k)
    o2 = oracle.attention(Q, K[:, perm], V[:, perm], n_q=n_q, n_k=n_k, head_dim=d, scale=0.5, batch=b)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-13)
    # one more feature column with q = 1 and k = 2 for every key adds 2*scale to every score
    one, two = np.uint16(0x3F80), np.uint16(0x4000)
    Qx = np.concatenate([Q, np.full((b, n_q, 1), one, np.uint16)], axis=2)
    Kx = np.concatenate([K, np.full((b, n_k, 1), two, np.uint16)], axis=2)
    Vx = np.concatenate([V, np.zeros((b, n_k, 1), np.uint16)], axis=2)
    o3 = oracle.attention(Qx, Kx, Vx, n_q=n_q, n_k=n_k, head_dim=d + 1, scale=0.5, batch=b)
    np.testing.assert_allclose(o3[:, :, :d], o, rtol=1e-13, atol=1e-13)


def test_attention_rows_and_strides_address_the_right_data():
    """Sampled rows equal the full result; padded leading dimensions and batch
    strides only move where rows are read."""
    b, n_q, n_k, d = 3, 7, 10, 8
    Q, K, V = _attn_inputs(18, b, n_q, n_k, d)
    full = oracle.attention(Q, K, V, n_q=n_q, n_k=n_k, head_dim=d, scale=0.3, batch=b)
    rows = np.array([[0, 0], [2, 6], [1, 3], [2, 0]])
    part = oracle.attention(Q, K, V, n_q=n_q, n_k=n_k, head_dim=d, scale=0.3, batch=b, rows=rows)
    assert np.array_equal(part, full[rows[:, 0], rows[:, 1]])
    pad = lambda X, ld: np.concatenate([X, np.full(X.shape[:2] + (ld - d,), np.uint16(0x7FC0))], axis=2)
    got = oracle.attention(pad(Q, 11), pad(K, 9), pad(V, 13), n_q=n_q, n_k=n_k, head_dim=d, scale=0.3, batch=b,
                           ldq=11, ldk=9, ldv=13)
    assert np.array_equal(got, full)
    with pytest.raises(IndexError):
        oracle.attention(Q, K, V, n_q=n_q, n_k=n_k, head_dim=d, scale=0.3, batch=b, rows=np.array([[3, 0]]))


# ------------------------------------------------------------- epilogue ---

def test_epilogue_identity_is_the_product():
    rng = np.random.default_rng(40)
    A = synth.draw(rng, (5, 7), "normal", 1.0)
    B = synth.draw(rng, (7, 3), "normal", 1.0)
    P = oracle.gemm(A, B, m=5, n=3, k=7)[0]
    assert np.array_equal(oracle.epilogue(P), P)
    assert np.array_equal(oracle.epilogue(P, 1.0, 0.0, np.full(P.shape, np.nan)), P)  # C not read at beta = 0


def test_epilogue_worked_example_by_hand():
    """A = I (2x2), B = [[1, 2], [3, 4]], C = [[10, 20], [30, 40]], bias = [0.5, -1]:
    2 * B - 1 * C + bias = [[-7.5, -17], [-23.5, -33]]."""
    A = oracle.round_to(np.eye(2), "bf16")
    B = oracle.round_to(np.array([[1.0, 2.0], [3.0, 4.0]]), "bf16")
    P = oracle.gemm(A, B, m=2, n=2, k=2)[0]
    out = oracle.epilogue(P, 2.0, -1.0, np.array([[10.0, 20.0], [30.0, 40.0]]), np.array([0.5, -1.0]))
    assert np.array_equal(out, np.array([[-7.5, -17.0], [-23.5, -33.0]]))


def test_epilogue_k0_and_batches():
    """K = 0: the product is zero, so the result is beta * C + bias in every
    batch (bias broadcast over rows and batches)."""
    A = np.zeros((3, 4, 0), dtype=np.uint16)
    B = np.zeros((3, 0, 5), dtype=np.uint16)
    P = oracle.gemm(A, B, m=4, n=5, k=0, batch=3, lda=1, ldb=5, stride_a=0, stride_b=0)
    C = np.arange(60, dtype=np.float64).reshape(3, 4, 5)
    bias = np.array([1.0, 2.0, 3.0, 4.0, 5.0])
    out = oracle.epilogue(P, 3.0, 0.5, C, bias)
    assert np.array_equal(out, 0.5 * C + bias[None, None, :])
