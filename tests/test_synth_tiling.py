"""The batch tiling of synthetic C4 cases (CPU): copy k of request r must be
request r read through index set k, which the oracle confirms row by row."""
import dataclasses

import numpy as np
import pytest

import oracle as oracle_mod
from synth import make_case, tile_requests


@pytest.fixture(scope="module")
def orc():
    oracle_mod.build()
    return oracle_mod.Oracle()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_tiled_copies_are_the_original_requests_through_their_sets(orc, kv):
    base = make_case(seq_lens=[900, 2600, 4001], n_q=[1, 3, 2], H=3, R=4, K=64, kv=kv, seed=17, index_sets=6)
    copies = 3
    tiled = tile_requests(base, copies)
    assert tiled.B == copies * base.B and tiled.T == copies * base.T
    assert tiled.meta["c4_sets"].shape == (2, copies * base.T, 64)
    out_t, lse_t, _ = orc.attention(tiled)
    sets = base.meta["c4_sets"]
    for k in range(copies):
        alone = dataclasses.replace(base, c4_indices=np.ascontiguousarray(sets[k]))
        out_k, lse_k, _ = orc.attention(alone)
        rows = slice(k * base.T, (k + 1) * base.T)
        assert np.array_equal(out_t[rows], out_k) and np.array_equal(lse_t[rows], lse_k)
    # every index any set names is backed: the oracle reads no poisoned row
    for j in range(tiled.meta["c4_sets"].shape[0]):
        o, l, _ = orc.attention(dataclasses.replace(tiled, c4_indices=np.ascontiguousarray(tiled.meta["c4_sets"][j])))
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def test_tiling_needs_whole_groups_of_sets():
    base = make_case(seq_lens=[900], n_q=1, H=2, R=4, K=16, seed=3, index_sets=5)
    with pytest.raises(ValueError):
        tile_requests(base, 2)
    assert tile_requests(base, 1) is base
