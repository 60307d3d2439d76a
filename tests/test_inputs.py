"""Seeded synthetic input generators: determinism and distribution shape."""

import numpy as np

from transformer_lm_step_gpt_amd import inputs as I


def test_batches_deterministic_and_shaped():
    for w in I.WORKLOADS.values():
        it1, it2 = I.batches(w, 2, 32), I.batches(w, 2, 32)
        for _ in range(2):
            (x1, y1), (x2, y2) = next(it1), next(it2)
            assert x1.dtype == np.int32 and x1.shape == (2, 32)
            assert np.array_equal(x1, x2) and np.array_equal(y1, y2)
            assert x1.min() >= 0 and x1.max() < w.model.vocab_size
            assert y1.min() >= 0 and y1.max() < w.model.vocab_size


def test_shifted_targets():
    for w in (I.CHAR_BF16, I.GPT2_124M):
        x, y = next(I.batches(w, 3, 50))
        assert np.array_equal(x.reshape(-1)[1:], y.reshape(-1)[:-1])


def test_zipf_eot_stream_structure():
    s = I.ZipfEotStream(7)
    t = s.take(200_000)
    assert t[0] == I.EOT_ID
    eot = np.flatnonzero(t == I.EOT_ID)
    lengths = np.diff(eot) - 1
    assert 450 < lengths.mean() < 750            # Geometric(1/600) on {1, 2, ...}
    assert lengths.min() >= 1
    words = t[t != I.EOT_ID]
    counts = np.bincount(words, minlength=I.EOT_ID)
    # Zipf(1.1): P(0)/P(1) = 2^1.1, and the top id holds ~ 1/H_{50256,1.1} of the mass
    r = counts[0] / counts[1]
    assert 1.8 < r < 2.5
    ranks = np.arange(1, I.EOT_ID + 1, dtype=np.float64)
    p0 = 1.0 / (ranks ** -1.1).sum()
    assert abs(counts[0] / len(words) - p0) < 0.01


def test_repeated_sequence_batch():
    x, y = I.repeated_sequence_batch(I.GPT2_124M, 4, 64)
    assert np.all(x == x[0]) and np.all(y == y[0])
    x1, y1 = next(I.batches(I.GPT2_124M, 1, 64))
    assert np.array_equal(x[0], x1[0])


def test_dirichlet_law():
    p = I.dirichlet_probs(I.CHAR_BF16)
    assert p.shape == (65,) and abs(p.sum() - 1) < 1e-12 and p.min() > 0
