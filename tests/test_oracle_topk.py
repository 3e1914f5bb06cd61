"""Pins of the C4 top-k oracle (oracle/topk.py), CPU only: brute force by
plain Python sorting on small rows, numpy's argpartition (an nth_element) on
rows whose threshold score is not tied, and closed forms."""
import numpy as np
import pytest

from oracle.topk import topk_select


def _brute(row, k):
    items = sorted(range(len(row)), key=lambda i: (-(float(row[i]) + 0.0), i))
    keep = sorted(items[:k])
    return keep + [-1] * (k - len(keep))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    T, ld, k = 5, 300, 40
    scores = rng.integers(-5, 6, (T, ld)).astype(np.float32)  # many ties
    scores[0, ::7] = -0.0
    scores[0, 1::7] = 0.0
    n = rng.integers(0, ld + 1, T)
    got = topk_select(scores, n, k)
    for t in range(T):
        assert got[t].tolist() == _brute(scores[t, :n[t]], k)


def test_matches_argpartition_without_threshold_ties():
    rng = np.random.default_rng(9)
    T, n, k = 4, 5000, 512
    scores = rng.standard_normal((T, n)).astype(np.float32)
    got = topk_select(scores, np.full(T, n), k)
    for t in range(T):
        part = np.sort(np.argpartition(-scores[t], k - 1)[:k])
        assert np.array_equal(got[t], part)


def test_closed_forms():
    k = 8
    eq = np.ones((1, 20), np.float32)
    assert topk_select(eq, [20], k)[0].tolist() == list(range(8))           # all tied: lowest indices
    inc = np.arange(20, dtype=np.float32)[None]
    assert topk_select(inc, [20], k)[0].tolist() == list(range(12, 20))     # increasing: the last k
    assert topk_select(inc, [5], k)[0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]  # fewer candidates than k
    assert topk_select(inc, [0], k)[0].tolist() == [-1] * 8
    z = np.array([[0.0, -0.0, 0.0, -1.0, -0.0]], np.float32)
    assert topk_select(z, [5], 2)[0].tolist() == [0, 1]                     # -0 ties with +0
    big = np.array([[3e38, -3e38, 1e-45, -1e-45, 2.0]], np.float32)
    assert topk_select(big, [5], 3)[0].tolist() == [0, 2, 4]
