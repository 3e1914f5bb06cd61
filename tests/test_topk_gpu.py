"""GPU parity of the C4 top-k selection (dsv4_c4_topk) against the oracle
(oracle/topk.py): the index lists must be identical (integer work)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as oracle_mod
from oracle.topk import topk_select
from synth import make_case
from tests import gpu_util as G

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def log(msg):
    print(msg, flush=True)


def _gpu(scores, n, k):
    from hybrid_sparse_mqa_amd import dsv4_c4_topk

    s = torch.from_numpy(np.ascontiguousarray(scores, np.float32)).cuda()
    c = torch.from_numpy(np.ascontiguousarray(n, np.int32)).cuda()
    out = dsv4_c4_topk(s, c, k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(scores, n, k, what):
    got = _gpu(scores, n, k)
    want = topk_select(scores, n, k)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} entries differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("k", [512, 64, 1])
def test_topk_ties_and_ragged_rows(k):
    rng = np.random.default_rng(k)
    T, ld = 12, 3000
    scores = rng.integers(-20, 21, (T, ld)).astype(np.float32)   # many ties at the threshold
    scores[1] = rng.standard_normal(ld).astype(np.float32)      # no ties
    scores[2, ::3] = -0.0                                        # -0 ties with +0
    scores[2, 1::3] = 0.0
    scores[3] = 7.0                                              # all tied
    n = np.array([ld, ld, ld, ld, 0, 1, k - 1 if k > 1 else 0, k, k + 1, 1000, 2999, 17], np.int32)
    log(f"topk: {T} rows, k={k}")
    _check(scores, n, k, f"k={k}")


def test_topk_million_token_rows():
    """Eight rows of 2^18 candidates (C4 entries of a 1M-token context)."""
    rng = np.random.default_rng(5)
    T, ld = 8, 1 << 18
    scores = rng.standard_normal((T, ld)).astype(np.float32)
    scores[1] = np.round(scores[1] * 4) / 4                      # heavy ties
    scores[2] = 1.0                                              # all tied
    n = np.full(T, ld, np.int32)
    n[3] = ld - 12345
    log("topk: 8 rows x 2^18 candidates")
    _check(scores, n, 512, "1M context")


def test_topk_feeds_the_attention():
    """Index lists selected on the GPU from random scores over each row's
    visible compressed entries, used as c4_indices: the attention matches the
    oracle's on the oracle's selection (the same lists)."""
    case = make_case(seq_lens=[3000, 4500], n_q=[1, 4], H=16, R=4, K=512, seed=6)
    rng = np.random.default_rng(6)
    pos = []
    for r in range(case.B):
        lo, hi = int(case.qo_indptr[r]), int(case.qo_indptr[r + 1])
        pos += [int(case.seq_lens[r]) - (hi - lo) + j for j in range(hi - lo)]
    n = np.array([(p + 1) // 4 for p in pos], np.int32)
    ld = int(n.max())
    scores = rng.standard_normal((case.T, ld)).astype(np.float32)
    # The generator backs only the compressed entries some row of the request
    # selected (the rest of the pool is poison): give the others a very low
    # score, so that every selection stays on backed entries (each row has at
    # least 512 of them).
    for r in range(case.B):
        lo, hi = int(case.qo_indptr[r]), int(case.qo_indptr[r + 1])
        backed = np.unique(case.c4_indices[lo:hi][case.c4_indices[lo:hi] >= 0])
        mask = np.ones(ld, bool)
        mask[backed] = False
        scores[lo:hi, mask] = -1e30
    got = _gpu(scores, n, 512)
    want = topk_select(scores, n, 512)
    assert np.array_equal(got, want)
    case = dataclasses.replace(case, c4_indices=got.astype(np.int32))
    out, lse = G.run_forward(case)
    ro, rl, _ = oracle_mod.Oracle().attention(dataclasses.replace(case, c4_indices=want.astype(np.int32)))
    G.compare(out, lse, ro, rl, what="topk -> attention")


# --------------------------------------------------------------------------
# Long rows (ld >= 32768): several workgroups per row build the first-digit
# histogram and compact the threshold digit's candidates; one finishes.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k", [512, 2048, 1])
def test_topk_long_rows_ragged(k):
    rng = np.random.default_rng(100 + k)
    ld = 1 << 17
    n = np.array([0, 1, k - 1, k, k + 1, 16383, 16384, 16385, 50000, ld - 1, ld], np.int32)
    n = np.clip(n, 0, ld)
    T = len(n)
    scores = rng.standard_normal((T, ld)).astype(np.float32)
    scores[5] = np.round(scores[5] * 8) / 8          # ties at every digit
    scores[6, ::2] = -0.0                             # -0 ties with +0
    scores[6, 1::2] = 0.0
    log(f"topk long rows: {T} x {ld}, k={k}")
    _check(scores, n, k, f"long k={k}")


@pytest.mark.parametrize("ld", [20000, 1 << 18], ids=["one-workgroup", "multi-workgroup"])
def test_topk_narrow_band(ld):
    """Scores 1 + 1e-4 N(0,1): nearly every candidate shares the first digit
    (far more than the 4096 the LDS list holds) without being tied, so the
    later digits and, for rounded values, the index tie-break decide."""
    rng = np.random.default_rng(7)
    T = 4
    scores = (1.0 + 1e-4 * rng.standard_normal((T, ld))).astype(np.float32)
    scores[1] = (1.0 + 1e-4 * np.round(rng.standard_normal(ld) * 16) / 16).astype(np.float32)
    n = np.array([ld, ld, ld - 1000, 9000], np.int32)
    log(f"topk narrow band ld={ld}")
    _check(scores, n, 512, f"narrow band ld={ld}")


@pytest.mark.parametrize("ld", [30000, 1 << 17], ids=["one-workgroup", "multi-workgroup"])
@pytest.mark.parametrize("n_bin", [4095, 4096, 4097])
def test_topk_threshold_digit_at_list_capacity(ld, n_bin):
    """Exactly n_bin candidates share the top first digit (values in
    [1, 1.125), some of them tied) and the rest lie far below: the threshold
    digit holds 4095, 4096 (the LDS list capacity) or 4097 candidates."""
    rng = np.random.default_rng(n_bin)
    T = 3
    scores = rng.uniform(-4.0, 0.5, (T, ld)).astype(np.float32)
    for t in range(T):
        where = rng.choice(ld, size=n_bin, replace=False)
        vals = rng.uniform(1.0, 1.125, n_bin).astype(np.float32)
        vals[: n_bin // 4] = np.float32(1.0625)  # a block of ties inside the digit
        scores[t, where] = vals
    n = np.full(T, ld, np.int32)
    log(f"topk threshold digit of {n_bin}, ld={ld}")
    _check(scores, n, 512, f"digit {n_bin} ld={ld}")


def test_topk_one_chunk_overflows_its_stage():
    """One 16384-candidate chunk holds 5000 equal scores above every other
    candidate (more survivors than a chunk stages), while the row's total
    stays under its list capacity: the row must still come out exact."""
    rng = np.random.default_rng(11)
    T, ld = 3, 1 << 18
    scores = rng.standard_normal((T, ld)).astype(np.float32)
    scores[0, 100:5100] = 5.0
    scores[1, 20000:25000] = 5.0
    scores[2, 20000:22000] = 5.0  # fits the stage: the normal path
    n = np.full(T, ld, np.int32)
    log("topk one chunk overflowing")
    for k in (512, 2048):
        _check(scores, n, k, f"stage overflow k={k}")


@pytest.mark.parametrize("k", [512, 2048, 1])
def test_topk_chunk_bound_layouts(k):
    """Rows whose full chunks offer very different bounds on the threshold
    digit: the best candidates all in one chunk, chunks offset from each
    other, the best candidates in the partial last chunk (which offers no
    bound), ties straddling the bound digit, and a plain row."""
    rng = np.random.default_rng(300 + k)
    T, ld = 6, (1 << 16) + 700
    scores = rng.standard_normal((T, ld)).astype(np.float32)
    scores[0] = np.linspace(-3.0, 3.0, ld, dtype=np.float32)          # increasing: the top K in the last chunk
    for c in range(ld // 16384 + 1):                                    # chunk c shifted by 0.75 c
        scores[1, 16384 * c:16384 * (c + 1)] += np.float32(0.75 * c)
    scores[2, 1 << 16:] = rng.uniform(10.0, 11.0, 700).astype(np.float32)  # the partial chunk holds the best
    scores[3] = np.round(scores[3] * 2) / 2                             # a few large tied digits
    scores[4, ::5] = np.float32(2.5)                                     # a tie block across every chunk
    n = np.array([ld, ld, ld, ld, ld, ld - 5000], np.int32)
    log(f"topk chunk bounds: {T} x {ld}, k={k}")
    _check(scores, n, k, f"chunk bounds k={k}")


@pytest.mark.parametrize("layout", ["offset-odd-stride", "aligned-ragged-width"])
def test_topk_unaligned_rows(layout):
    """Score rows the long-row path cannot read 16 bytes at a time: a view
    one column into a wider tensor (odd row stride, unaligned rows), and
    aligned rows whose width is not a multiple of 4 (the last vector would
    reach past the row's last score).  One score at a time there; the result
    must be the same."""
    from hybrid_sparse_mqa_amd import dsv4_c4_topk

    rng = np.random.default_rng(17)
    T, ld = 4, (1 << 16) + 2
    wide = rng.standard_normal((T, ld + 2)).astype(np.float32)
    wide[2] = np.round(wide[2] * 4) / 4  # ties
    n = np.array([ld, ld - 1, ld - 2, 40000], np.int32)
    full = torch.from_numpy(wide).cuda()
    if layout == "offset-odd-stride":
        full = full[:, : ld + 1]
        full = torch.as_strided(full.contiguous(), (T, ld), (ld + 1, 1), 1)
        host = full.cpu().numpy()
        assert full.data_ptr() % 16 != 0 and full.stride(0) % 4 != 0
    else:
        full = full[:, :ld]
        host = wide[:, :ld]
        assert full.data_ptr() % 16 == 0 and full.stride(0) % 4 == 0 and ld % 4 != 0
    for k in (512, 2048):
        got = dsv4_c4_topk(full, torch.from_numpy(n).cuda(), k)
        torch.cuda.synchronize()
        want = topk_select(np.ascontiguousarray(host), n, k)
        assert np.array_equal(got.cpu().numpy(), want), f"{layout} k={k}"
