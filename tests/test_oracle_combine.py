"""Pins for the oracle's split-K merge (CPU only): merging the softmax
statistics of the pieces of a key range must give the attention over the
whole range -- an identity of exp(a + b) = exp(a) exp(b) -- for any split,
empty pieces and single-token pieces included, and a merge that forgets the
rescaling must fail it."""
import numpy as np
import pytest

from oracle import attention as oatt


def _pieces(rng, L):
    cuts = np.sort(rng.integers(0, L + 1, size=int(rng.integers(0, 6))))
    bounds = [0] + cuts.tolist() + [L]
    return list(zip(bounds[:-1], bounds[1:]))


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_any_split_equals_whole_range_attention(seed):
    rng = np.random.default_rng(300 + seed)
    D = int(rng.choice([8, 64, 128]))
    L = int(rng.integers(1, 400))
    q = rng.standard_normal(D) * rng.uniform(0.1, 4.0)
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    scale = 1.0 / np.sqrt(D)
    want = oatt.attend(q, K, V, scale)
    for _ in range(5):
        parts = [oatt.partial_attend(q, K[a:b], V[a:b], scale) for a, b in _pieces(rng, L)]
        got = oatt.combine_partials(parts)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_single_token_pieces_and_large_score_gaps():
    rng = np.random.default_rng(7)
    D, L = 16, 40
    q = rng.standard_normal(D) * 30.0          # scores far apart: exp(m_i - M) spans many decades
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    want = oatt.attend(q, K, V, 1.0)
    parts = [oatt.partial_attend(q, K[i:i + 1], V[i:i + 1], 1.0) for i in range(L)]
    assert np.allclose(oatt.combine_partials(parts), want, rtol=1e-12, atol=1e-12)
    assert np.allclose(oatt.combine_partials(parts[::-1]), want, rtol=1e-12, atol=1e-12)


def test_partial_of_empty_piece_and_of_whole_range():
    rng = np.random.default_rng(8)
    q, K, V = rng.standard_normal(8), rng.standard_normal((5, 8)), rng.standard_normal((5, 8))
    m, l, acc = oatt.partial_attend(q, K[:0], V[:0], 0.5)
    assert m == -np.inf and l == 0.0 and not acc.any()
    m, l, acc = oatt.partial_attend(q, K, V, 0.5)
    assert np.allclose(acc / l, oatt.attend(q, K, V, 0.5), rtol=1e-14)
    assert m == np.max(K @ q * 0.5)


def test_a_merge_without_the_rescaling_fails_the_identity():
    rng = np.random.default_rng(9)
    D, L = 32, 64
    q = rng.standard_normal(D) * 3.0
    K, V = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    want = oatt.attend(q, K, V, 1.0 / np.sqrt(D))
    parts = [oatt.partial_attend(q, K[a:b], V[a:b], 1.0 / np.sqrt(D)) for a, b in ((0, 20), (20, 64))]
    wrong = sum(acc for _, _, acc in parts) / sum(l for _, l, _ in parts)   # planted: no exp(m_i - M)
    assert not np.allclose(wrong, want, rtol=1e-6)
    assert np.allclose(oatt.combine_partials(parts), want, rtol=1e-12)
