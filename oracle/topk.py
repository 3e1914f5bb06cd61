"""C4 top-k selection, the oracle (TEST INFRASTRUCTURE ONLY: only tests/ and
bench.py's CPU baseline use it; the product path never imports it).

The step in front of the C4 attention (the DSV4 overview page, "what V4
changed": the indexer keeps the top 512 compressed entries per query; its
kernel section names the Lightning TopK kernel): given each row's scores over
its candidate compressed entries 0 .. n-1, keep the K entries with the
highest scores.  The pages do not say how equal scores are broken; the
reading taken here: a lower index wins, and -0.0 equals +0.0.  The kept
indices are returned in ascending order, then -1 up to width K (rows with
fewer than K candidates keep all of them).  Scores must be finite.

Written as the definition: a stable sort of the candidates by descending
score (numpy's lexsort, index as the secondary key), the first K taken, then
sorted by index.  Pinned by tests/test_oracle_topk.py (brute force by plain
Python sorting, numpy's argpartition where no tie sits at the threshold,
closed forms).
"""
from __future__ import annotations

import numpy as np


def topk_select(scores: np.ndarray, n_cand: np.ndarray, k: int) -> np.ndarray:
    """scores f32 [T, ld], n_cand i32 [T] (0 <= n <= ld) -> indices i32 [T, k]."""
    scores = np.asarray(scores, np.float32)
    T = scores.shape[0]
    out = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = int(n_cand[t])
        s = scores[t, :n].astype(np.float64) + 0.0  # -0.0 + 0.0 == +0.0
        idx = np.arange(n)
        order = np.lexsort((idx, -s))  # descending score, then ascending index
        keep = np.sort(order[:k])
        out[t, :len(keep)] = keep
    return out
