"""The no-allocation forward entry point (dsv4_attn_forward_noalloc, -m gpu).

Called through the C ABI, it must return exactly what dsv4_attn_forward
returns (same kernels and plan; only the split partials live elsewhere), on
two calls in a row whose second input is smaller than the first (the static
scratch keeps the first call's partials, which the second must not use),
refuse calls whose partials exceed the static scratch before launching
anything, and stay correct when captured into a HIP graph.
"""
import pytest
import torch

import oracle
from synth import make_case
from tests import gpu_util as G

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def both(case):
    from hybrid_sparse_mqa_amd import dsv4_attn_forward, dsv4_attn_forward_noalloc

    g = G.to_gpu(case)
    args = (g["q"], g["swa_pool"], g["swa_page_table"], g["extra_pool"], g["extra_page_table"], g["c4_indices"],
            g["seq_lens"], g["qo_indptr"], g["sink"], case.R, case.W, case.scale)
    ref = dsv4_attn_forward(*args)
    out = torch.full_like(ref[0], 3.0)
    lse = torch.full_like(ref[1], 3.0)
    dsv4_attn_forward_noalloc(*args, out=out, lse=lse)
    torch.cuda.synchronize()
    return ref, (out, lse)


def plan_splits(case):
    from hybrid_sparse_mqa_amd import dsv4_attn_plan

    p_extra = 0 if case.extra_page_table is None else case.extra_page_table.shape[1]
    return dsv4_attn_plan(case.T, case.H, case.R, case.W, case.K, p_extra, kv_fp8=case.kv == "fp8")[0]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_matches_forward_then_smaller_call(kv):
    big = make_case(seq_lens=[9000, 4000, 700, 3000], n_q=[1, 4, 2, 1], H=64, R=4, seed=21, kv=kv)
    small = make_case(seq_lens=[300, 40], n_q=[2, 1], H=16, R=128 if kv == "bf16" else 4, seed=22, kv=kv)
    assert plan_splits(big) > 1  # the first call uses the scratch
    for case in (big, small):
        (ro, rl), (out, lse) = both(case)
        assert torch.equal(out, ro) and torch.equal(lse, rl), case.name
        ro64, rl64, _ = oracle.Oracle().attention(case)
        G.compare(out, lse, ro64, rl64, what=f"noalloc {kv} {case.name}")


def test_noalloc_refuses_partials_beyond_scratch():
    from hybrid_sparse_mqa_amd import (Dsv4Error, dsv4_attn_forward_noalloc, dsv4_attn_noalloc_scratch_bytes,
                                       dsv4_attn_set_split_keys)

    cap = dsv4_attn_noalloc_scratch_bytes()
    assert cap == 32 << 20
    # 16 rows x 128 heads of C4 decode in 32-key splits: 20 splits per row,
    # 16 x 20 x 128 x 1028 bytes = 42 MB of partials.
    case = make_case(seq_lens=[6000] * 16, n_q=1, H=128, R=4, seed=23)
    g = G.to_gpu(case)
    out = torch.full((case.T, case.H, 512), 5.0, dtype=torch.bfloat16, device="cuda")
    dsv4_attn_set_split_keys(32)
    try:
        splits = plan_splits(case)
        assert case.T * splits * case.H * 1028 > cap, splits
        with pytest.raises(Dsv4Error, match="ERR_WORKSPACE"):
            dsv4_attn_forward_noalloc(g["q"], g["swa_pool"], g["swa_page_table"], g["extra_pool"],
                                      g["extra_page_table"], g["c4_indices"], g["seq_lens"], g["qo_indptr"],
                                      g["sink"], case.R, case.W, case.scale, out=out, return_lse=False)
    finally:
        dsv4_attn_set_split_keys(0)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)  # nothing was launched


def test_noalloc_under_graph_capture():
    from hybrid_sparse_mqa_amd import dsv4_attn_forward_noalloc

    case = make_case(seq_lens=[3000, 5000, 700], n_q=[1, 4, 2], H=64, R=4, seed=24)
    assert plan_splits(case) > 1
    (ro, rl), _ = both(case)
    g = G.to_gpu(case)
    out = torch.zeros_like(ro)
    lse = torch.zeros_like(rl)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            dsv4_attn_forward_noalloc(g["q"], g["swa_pool"], g["swa_page_table"], g["extra_pool"],
                                      g["extra_page_table"], g["c4_indices"], g["seq_lens"], g["qo_indptr"],
                                      g["sink"], case.R, case.W, case.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(lse, rl), rep
        both(make_case(seq_lens=[2000] * 9, n_q=1, H=64, R=128, seed=25))  # other noalloc work in between
