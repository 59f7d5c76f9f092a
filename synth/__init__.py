"""Seeded synthetic inputs for the tiled GEMM/BMM workloads.

This module only draws random numbers and encodes them as 16-bit floating
point bit patterns.  It holds none of the matrix-multiply arithmetic: both the
HIP path (through the tests and the benchmark) and the CPU oracle receive the
very same arrays from here, and neither side's code lives here.

Recipe (the pages fix no generator, seed layout or encoding; these are the
readings this project takes):

* ``numpy.random.default_rng(seed)`` (PCG64).  Each array is drawn whole, in
  C order, in the order its workload lists it; large arrays are drawn in
  contiguous chunks, which yields the same stream as one draw.
* Uniform on [lo, hi): ``lo + (hi - lo) * rng.random()``.  Normal with
  standard deviation s: ``s * rng.standard_normal()``.
* float64 draws are rounded to float32 (round-to-nearest-even) and then to
  bf16 by round-to-nearest-even using torch's own conversion; fp16 inputs are
  rounded from float64 by numpy's conversion.  Rounding may turn a value just
  below ``hi`` into ``hi``; tolerances use the observed maxima, so this is
  harmless.

The workloads are the GEMM shapes the pages tune for (square, ragged, tall-thin
inference) and the two batched products of an attention head
(p1 "Triton Optimization Reference", intro and section 3; p2 "Optimize Triton
Block Parameters", Performance requirements, shape-specific tuning).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

_CHUNK = 1 << 22  # elements per draw; any value gives the same stream


def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _encode(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return _f32_to_bf16_bits(x64.astype(np.float32))
    if dtype == "fp16":
        return x64.astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown input dtype {dtype!r}")


def draw(rng: np.random.Generator, shape, dist: str, a: float, b: float = 0.0,
         dtype: str = "bf16") -> np.ndarray:
    """Draw an array of 16-bit float bit patterns (uint16) of ``shape``.

    ``dist`` is "uniform" (on [a, b)), "normal" (std a) or "int" (integers in
    [a, b], inclusive, exactly representable).
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _CHUNK):
        cnt = min(_CHUNK, n - lo)
        if dist == "uniform":
            x = a + (b - a) * rng.random(cnt)
        elif dist == "normal":
            x = a * rng.standard_normal(cnt)
        elif dist == "int":
            x = rng.integers(int(a), int(b) + 1, size=cnt).astype(np.float64)
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        out[lo:lo + cnt] = _encode(x, dtype)
    return out.reshape(shape)


def bits_to_float(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Widen bit patterns to float32 (for host-side inspection only)."""
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


@dataclasses.dataclass
class Problem:
    """One GEMM or BMM call: C[b] = op(A[b]) @ op(B[b]) with row-major storage."""
    name: str
    A: np.ndarray                 # uint16 bit patterns, stored shape
    B: np.ndarray
    trans_a: int
    trans_b: int
    m: int
    n: int
    k: int
    batch: int = 1
    in_dtype: str = "bf16"
    out_dtype: str = "fp32"
    lda: int = 0
    ldb: int = 0
    ldc: int = 0
    stride_a: int = 0
    stride_b: int = 0
    stride_c: int = 0

    def __post_init__(self):
        if not self.lda:
            self.lda = self.m if self.trans_a else self.k
        if not self.ldb:
            self.ldb = self.k if self.trans_b else self.n
        if not self.ldc:
            self.ldc = self.n
        if self.batch > 1:
            if not self.stride_a:
                self.stride_a = (self.k if self.trans_a else self.m) * self.lda
            if not self.stride_b:
                self.stride_b = (self.n if self.trans_b else self.k) * self.ldb
            if not self.stride_c:
                self.stride_c = self.m * self.ldc

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k * self.batch


# ---------------------------------------------------------------------------
# The five workloads.  Sizes, distributions and seeds are the ones the
# project's benchmark configurations name; layouts follow the readings listed
# in the design notes (row-major op letters; NT = B stored N x K).
# ---------------------------------------------------------------------------

def square_256(seed: int = 0) -> List[Problem]:
    rng = np.random.default_rng(seed)
    A = draw(rng, (256, 256), "uniform", -1.0, 1.0)
    B = draw(rng, (256, 256), "uniform", -1.0, 1.0)
    return [Problem("square_256_nn", A, B, 0, 0, 256, 256, 256)]


def ragged_1000(seed: int = 1) -> List[Problem]:
    """The same two stored 1000x1000 arrays read under all four transposes."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (1000, 1000), "uniform", -1.0, 1.0)
    B = draw(rng, (1000, 1000), "uniform", -1.0, 1.0)
    out = []
    for ta in (0, 1):
        for tb in (0, 1):
            tag = ("T" if ta else "N") + ("T" if tb else "N")
            out.append(Problem(f"ragged_1000_{tag.lower()}", A, B, ta, tb, 1000, 1000, 1000))
    return out


def skinny_16(seed: int = 2, out_dtype: str = "bf16") -> List[Problem]:
    """M=16 activations against an N x K weight matrix (B stored N x K)."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (16, 8192), "normal", 1.0)
    B = draw(rng, (8192, 8192), "normal", 0.02)
    return [Problem("skinny_16x8192x8192_nt", A, B, 0, 1, 16, 8192, 8192, out_dtype=out_dtype)]


def attention_bmm(seed: int = 3, batch: int = 128, seq: int = 2048, head: int = 128) -> List[Problem]:
    """S = Q K^T and O = P V for ``batch`` heads; P is independent synthetic data."""
    rng = np.random.default_rng(seed)
    Q = draw(rng, (batch, seq, head), "normal", 1.0)
    K = draw(rng, (batch, seq, head), "normal", 1.0)
    P = draw(rng, (batch, seq, seq), "uniform", 0.0, 1.0 / 2048.0)
    V = draw(rng, (batch, seq, head), "normal", 1.0)
    s = Problem(f"attn_s_b{batch}_{seq}x{seq}x{head}_nt", Q, K, 0, 1, seq, seq, head, batch=batch)
    o = Problem(f"attn_o_b{batch}_{seq}x{head}x{seq}_nn", P, V, 0, 0, seq, head, seq, batch=batch)
    return [s, o]


def square_8192(seed: int = 4, out_dtype: str = "bf16", layout: str = "nn") -> List[Problem]:
    """8192^3 with both operands drawn N(0, 1); ``layout`` picks op(A) op(B)
    (the stored arrays are square, so every layout reads the same draws)."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (8192, 8192), "normal", 1.0)
    B = draw(rng, (8192, 8192), "normal", 1.0)
    ta, tb = int(layout[0] == "t"), int(layout[1] == "t")
    return [Problem(f"square_8192_{layout}", A, B, ta, tb, 8192, 8192, 8192, out_dtype=out_dtype)]


def long_k(seed: int = 10, m: int = 1024, n: int = 1024, k: int = 65536, out_dtype: str = "bf16") -> List[Problem]:
    """A product with few output tiles and a long K (64 tiles of 128 x 128 on
    256 compute units): the shape split-K exists for."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (m, k), "normal", 1.0)
    B = draw(rng, (k, n), "normal", 1.0)
    return [Problem(f"long_k_{m}x{n}x{k}_nn", A, B, 0, 0, m, n, k, out_dtype=out_dtype)]


@dataclasses.dataclass
class AttnProblem:
    """O = softmax(scale * Q K^T) V for ``batch`` heads, row-major with the head
    dimension contiguous: Q [batch, n_q, d], K and V [batch, n_k, d]."""
    name: str
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    n_q: int
    n_k: int
    d: int
    scale: float
    batch: int = 1
    out_dtype: str = "fp32"

    @property
    def flops(self) -> float:
        """Two n_q x n_k x d products per head (the softmax's arithmetic is not counted)."""
        return 4.0 * self.batch * self.n_q * self.n_k * self.d


def attention_fwd(seed: int = 5, batch: int = 128, seq: int = 2048, head: int = 128,
                  out_dtype: str = "fp32") -> AttnProblem:
    """Fused attention forward pass on the attention-shaped workload's sizes:
    Q, K, V ~ N(0, 1) drawn in that order from one stream, scale 1/sqrt(head)."""
    rng = np.random.default_rng(seed)
    Q = draw(rng, (batch, seq, head), "normal", 1.0)
    K = draw(rng, (batch, seq, head), "normal", 1.0)
    V = draw(rng, (batch, seq, head), "normal", 1.0)
    return AttnProblem(f"attn_fwd_b{batch}_{seq}x{seq}_d{head}", Q, K, V, seq, seq, head, 1.0 / float(np.sqrt(head)),
                       batch, out_dtype)


def attention_rows(seed: int, batch: int, n_q: int, count: int = 512,
                   edges: Tuple[int, ...] = (0, 31, 32, 63, 64, 127, 128)) -> np.ndarray:
    """Seeded (b, i) query rows: ``count`` uniform draws plus tile-edge rows in
    the first and last head."""
    rng = np.random.default_rng(2000 + seed)
    r = np.stack([rng.integers(0, batch, count), rng.integers(0, n_q, count)], 1)
    e = [i for i in edges if i < n_q] + [n_q - 1]
    extra = [[b, i] for b in {0, batch - 1} for i in e]
    return np.concatenate([r, np.array(extra, dtype=np.int64)]).astype(np.int64)


WORKLOADS = {
    "square_256": square_256,
    "ragged_1000": ragged_1000,
    "skinny_16": skinny_16,
    "attention_bmm": attention_bmm,
    "square_8192": square_8192,
}


@dataclasses.dataclass
class GroupedProblem:
    """A ragged list of products sharing N and K, as in a mixture-of-experts
    layer: tokens X [T, K] sorted by expert, expert e owns rows
    [offsets[e], offsets[e+1]) and multiplies them by its weights W[e] [K, N]
    (NN, row-major); outputs go to the matching rows of Y [T, N]."""
    name: str
    X: np.ndarray
    W: np.ndarray
    counts: np.ndarray
    n: int
    k: int
    out_dtype: str = "bf16"

    @property
    def offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.counts)]).astype(np.int64)

    @property
    def flops(self) -> float:
        return 2.0 * float(self.counts.sum()) * self.n * self.k

    def algorithmic_bytes(self, out_size: int) -> float:
        """X and the weights read once, Y written once."""
        t = float(self.counts.sum())
        return 2.0 * t * self.k + 2.0 * len(self.counts) * self.k * self.n + out_size * t * self.n


def grouped_moe(seed: int = 6, experts: int = 32, tokens: int = 8192, k: int = 1024, n: int = 1024,
                out_dtype: str = "bf16") -> GroupedProblem:
    """Ragged expert GEMMs: expert loads from a multinomial over Dirichlet(1)
    weights (uneven, some experts may get no tokens), X ~ N(0, 1), W ~ N(0, 1/K)."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(tokens, rng.dirichlet(np.ones(experts))).astype(np.int64)
    X = draw(rng, (tokens, k), "normal", 1.0)
    W = draw(rng, (experts, k, n), "normal", 1.0 / float(np.sqrt(k)))
    return GroupedProblem(f"grouped_moe_e{experts}_t{tokens}_k{k}_n{n}", X, W, counts, n, k, out_dtype)


def sample_indices(seed: int, batch: int, m: int, n: int, count: int = 4096,
                   edges: Tuple[int, ...] = (0, 63, 64, 127, 128, 255, 256)) -> np.ndarray:
    """Seeded (b, i, j) triples: ``count`` uniform draws plus tile-edge points.

    Edge points are every pair of {edges, M-1} x {edges, N-1} (clipped to the
    matrix) in the first and last batch.
    """
    rng = np.random.default_rng(1000 + seed)
    b = rng.integers(0, batch, size=count)
    i = rng.integers(0, m, size=count)
    j = rng.integers(0, n, size=count)
    ei = sorted({e for e in edges if e < m} | {m - 1}) if m else []
    ej = sorted({e for e in edges if e < n} | {n - 1}) if n else []
    extra = [(bb, ii, jj) for bb in sorted({0, batch - 1}) for ii in ei for jj in ej]
    tri = np.stack([b, i, j], axis=1).astype(np.int64)
    if extra:
        tri = np.concatenate([tri, np.asarray(extra, dtype=np.int64)], axis=0)
    return np.ascontiguousarray(tri)
