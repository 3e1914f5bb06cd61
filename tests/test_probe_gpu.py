"""The plain streaming-read timing helper (dsv4_read_probe) on the GPU: it
runs over ragged sizes and workgroup counts and leaves its sink untouched
(the sink is written only if the folded bytes hit one fixed constant, which
a constant fill cannot produce)."""
import pytest
import torch

from hybrid_sparse_mqa_amd import dsv4_read_probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096, 3), ((1 << 20) + 48, 1024), (24 << 20, 1024), (24 << 20, 7)])
def test_read_probe_runs_and_leaves_sink(nbytes, wgs):
    buf = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    sink = torch.full((16,), 0xEE, dtype=torch.uint8, device="cuda")
    dsv4_read_probe(buf, nbytes, wgs, sink)
    torch.cuda.synchronize()
    assert bool((sink == 0xEE).all())


def test_read_probe_rejects_oversized_reads():
    buf = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        dsv4_read_probe(buf, 2048, 4, sink)
