"""The seeded input generator: deterministic, chunk-invariant, right shapes and spread."""
import numpy as np
import pytest

import synth


def test_same_seed_same_bits_and_chunking_does_not_change_the_stream(monkeypatch):
    a = synth.draw(np.random.default_rng(3), (300, 500), "normal", 1.0)
    monkeypatch.setattr(synth, "_CHUNK", 777)
    b = synth.draw(np.random.default_rng(3), (300, 500), "normal", 1.0)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    c = synth.draw(np.random.default_rng(3), (300, 500), "uniform", -1.0, 1.0)
    monkeypatch.setattr(synth, "_CHUNK", 1 << 22)
    d = synth.draw(np.random.default_rng(3), (300, 500), "uniform", -1.0, 1.0)
    assert np.array_equal(c, d)


@pytest.mark.parametrize("dist,a,b,lo,hi,mean,std", [
    ("uniform", -1.0, 1.0, -1.0, 1.0, 0.0, 1 / np.sqrt(3)),
    ("uniform", 0.0, 1 / 2048, 0.0, 1 / 2048, 0.5 / 2048, 1 / 2048 / np.sqrt(12)),
    ("normal", 0.02, 0.0, -np.inf, np.inf, 0.0, 0.02),
])
def test_distributions(dist, a, b, lo, hi, mean, std):
    x = synth.bits_to_float(synth.draw(np.random.default_rng(0), (200_000,), dist, a, b)).astype(np.float64)
    assert x.min() >= lo and x.max() <= hi
    assert abs(x.mean() - mean) < 0.02 * std + 1e-12
    assert abs(x.std() - std) < 0.02 * std


def test_integer_draws_are_exact():
    x = synth.bits_to_float(synth.draw(np.random.default_rng(0), (10_000,), "int", -8, 8))
    assert np.array_equal(x, np.round(x)) and x.min() == -8 and x.max() == 8
    h = synth.bits_to_float(synth.draw(np.random.default_rng(0), (10_000,), "int", -8, 8, dtype="fp16"), "fp16")
    assert np.array_equal(h, x)


def test_small_workload_shapes_and_layouts():
    (p,) = synth.square_256()
    assert p.A.shape == (256, 256) and (p.trans_a, p.trans_b, p.out_dtype) == (0, 0, "fp32")
    probs = synth.ragged_1000()
    assert [(q.trans_a, q.trans_b) for q in probs] == [(0, 0), (0, 1), (1, 0), (1, 1)]
    assert all(q.A is probs[0].A and q.B is probs[0].B for q in probs)
    s, o = synth.attention_bmm(batch=2, seq=64, head=32)
    assert (s.m, s.n, s.k, s.trans_b, s.ldb, s.stride_b, s.stride_c) == (64, 64, 32, 1, 32, 64 * 32, 64 * 64)
    assert (o.m, o.n, o.k, o.trans_b, o.lda, o.stride_a, o.stride_b) == (64, 32, 64, 0, 64, 64 * 64, 64 * 32)


def test_sample_indices_are_seeded_in_range_and_include_edges():
    t = synth.sample_indices(4, 3, 300, 1000)
    assert t.shape[1] == 3 and t.shape[0] > 4096
    assert np.array_equal(t, synth.sample_indices(4, 3, 300, 1000))
    assert t[:, 0].max() < 3 and t[:, 1].max() < 300 and t[:, 2].max() < 1000 and t.min() >= 0
    rows = {tuple(r) for r in t.tolist()}
    assert (0, 299, 999) in rows and (2, 0, 0) in rows and (0, 256, 128) in rows
