"""Bit-exact key sets of the split kernels that dsv4_attn_forward runs (-m gpu).

The library's key-recording hook (dsv4_attn_debug_keys) makes a forward call
launch the recording build of its split kernel, which stores, for every work
item (row, head block, split) and every key of the split, the address of the
KV row it copied into LDS or registers, and, for the 32- and 64-head kernels,
the valid-key mask of every 32-key tile.  These tests decode the addresses
back to (pool, physical slot) and compare them, in the kernel's own key order,
with the oracle's gather (canonical slot lists) plus the row's C4 index list
(for the position of unused entries):

* the 32- and 64-head and FP8 kernels walk the compressed entries first
  (C4: the whole index list, -1 entries reading the zero row and masked
  out; C128: entries 0 .. visible-1), then the window ascending;
* the 16-head kernel walks the window first, then the compressed entries in
  the same way.

Keys past a split's end up to its last tile must read the zero row; the
valid-key masks must mark exactly the used keys.  The recording build must
also produce output and lse bit-identical to the plain build.
"""
import numpy as np
import pytest
import torch

import oracle as oracle_mod
from synth import make_case, make_config
from tests import gpu_util as G
from tests.test_parity_gpu import SMALL, SMALL_IDS, small_case

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SENTINEL = 0x5A5A5A5A5A5A5A5A
MASK_SENTINEL = 0xA5A5A5A5
H16, H32, ROLES, H64, FP8, FP8_H32 = 1, 2, 3, 4, 5, 6
FP8_KERNELS = (FP8, FP8_H32)
TILE = {H16: 16, H32: 32, ROLES: 32, H64: 32, FP8: 32, FP8_H32: 32}
HEADS = {H16: 16, H32: 32, ROLES: 32, H64: 64, FP8: 64, FP8_H32: 32}
COMPRESSED_FIRST = {H16: False, H32: True, ROLES: True, H64: True, FP8: True, FP8_H32: True}
MASKED = {H32, ROLES, H64}


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.Oracle()


def log(msg):
    print(msg, flush=True)


def record(case, kernel=0, split_keys=0, g=None):
    """Run the forward with the recording hook; returns (keys [T, hb, S, chunk]
    uint64, masks [T, hb, S, 32] uint32, plan (splits, chunk, kernel), g,
    out, lse)."""
    from hybrid_sparse_mqa_amd import (dsv4_attn_debug_keys, dsv4_attn_plan, dsv4_attn_set_kernel,
                                       dsv4_attn_set_split_keys)

    g = G.to_gpu(case) if g is None else g
    assert kernel == 0 or (kernel in FP8_KERNELS) == (case.kv == "fp8"), "a forced variant of the other format"
    dsv4_attn_set_kernel(kernel)
    dsv4_attn_set_split_keys(split_keys)
    try:
        p_extra = 0 if case.extra_page_table is None else case.extra_page_table.shape[1]
        splits, chunk, kern = dsv4_attn_plan(case.T, case.H, case.R, case.W, case.K, p_extra,
                                             kv_fp8=case.kv == "fp8")
        hb = -(-case.H // HEADS[kern])
        keys = torch.full((case.T, hb, splits, chunk), SENTINEL, dtype=torch.int64, device="cuda")
        masks = torch.full((case.T, hb, splits, 32), MASK_SENTINEL - (1 << 32), dtype=torch.int32, device="cuda")
        dsv4_attn_debug_keys(keys, masks)
        try:
            out, lse = G.run_forward(case, g)
        finally:
            dsv4_attn_debug_keys(None)
        plain_out, plain_lse = G.run_forward(case, g)
    finally:
        dsv4_attn_set_kernel(0)
        dsv4_attn_set_split_keys(0)
    assert torch.equal(out, plain_out) and torch.equal(lse, plain_lse), "recording build changed the result"
    k = keys.cpu().numpy().view(np.uint64)
    m = masks.cpu().numpy().view(np.uint32)
    return k, m, (splits, chunk, kern), g, out, lse


class Decoder:
    """Device row address -> ("swa" | "ext", slot) or "zero"."""

    def __init__(self, case, g):
        self.fp8 = case.kv == "fp8"
        self.pools = []
        for name in ("swa", "ext"):
            t = g["swa_pool" if name == "swa" else "extra_pool"]
            if t is None:
                continue
            base = t.data_ptr()
            size = t.numel() * t.element_size()
            row = 149504 if self.fp8 else t.stride(0) * t.element_size()
            self.pools.append((name, base, size, row))
        self.zero = None

    def __call__(self, addr):
        addr = int(addr)
        for name, base, size, row in self.pools:
            if base <= addr < base + size:
                off = addr - base
                if self.fp8:
                    page, rem = divmod(off, 149504)
                    rec, r2 = divmod(rem, 576)
                    assert r2 == 0 and rec < 256, f"address {addr:#x} is not a record start"
                    return (name, page * 256 + rec)
                slot, r2 = divmod(off, row)
                assert r2 == 0, f"address {addr:#x} is not a row start"
                return (name, slot)
        if self.zero is None:
            self.zero = addr
        assert addr == self.zero, f"two different addresses outside the pools: {self.zero:#x}, {addr:#x}"
        return "zero"


def check_keys(orc, case, kernel=0, split_keys=0, what=""):
    keys, masks, (splits, chunk, kern), g, _, _ = record(case, kernel, split_keys)
    if kernel:
        assert kern == kernel
    dec = Decoder(case, g)
    tile = TILE[kern]
    hb_n = keys.shape[1]
    for t in range(case.T):
        exp = G.expected_keys(orc, case, t, COMPRESSED_FIRST[kern])
        n = len(exp)
        for s in range(splits):
            k0 = s * chunk
            n_here = max(0, min(n, k0 + chunk) - k0)
            n_tiles = -(-n_here // tile)
            for hb in range(hb_n):
                rec = keys[t, hb, s]
                got = [dec(a) for a in rec[:n_tiles * tile]]
                want = [("zero" if e is None else e) for e in exp[k0:k0 + n_here]] + ["zero"] * (n_tiles * tile - n_here)
                if got != want:
                    bad = next(i for i in range(len(want)) if got[i] != want[i])
                    raise AssertionError(f"{what} row {t} hb {hb} split {s}: key {bad} read {got[bad]}, "
                                         f"expected {want[bad]} (chunk {chunk}, n_here {n_here}, kernel {kern})")
                assert np.all(rec[n_tiles * tile:] == np.uint64(SENTINEL)), f"{what}: keys past the last tile written"
                if kern in MASKED:
                    for j in range(32):
                        if j < n_tiles:
                            bits = sum(1 << b for b in range(32)
                                       if j * 32 + b < n_here and exp[k0 + j * 32 + b] is not None)
                            assert int(masks[t, hb, s, j]) == bits, \
                                f"{what} row {t} hb {hb} split {s} tile {j}: mask {int(masks[t, hb, s, j]):#x} != {bits:#x}"
                        else:
                            assert int(masks[t, hb, s, j]) == MASK_SENTINEL
    return splits, chunk, kern


BF16_CASES = [i for i, c in enumerate(SMALL) if c[5] == "bf16"]
FP8_CASES = [i for i, c in enumerate(SMALL) if c[5] == "fp8"]


@pytest.mark.parametrize("kernel", [0, H16, H32, ROLES, H64])
@pytest.mark.parametrize("i", BF16_CASES, ids=[SMALL_IDS[i] for i in BF16_CASES])
def test_keys_small_bf16(orc, i, kernel):
    log(f"keys {SMALL_IDS[i]} kernel={kernel}")
    check_keys(orc, small_case(i), kernel, what=SMALL_IDS[i])


@pytest.mark.parametrize("kernel", [0, FP8, FP8_H32])
@pytest.mark.parametrize("i", FP8_CASES, ids=[SMALL_IDS[i] for i in FP8_CASES])
def test_keys_small_fp8(orc, i, kernel):
    log(f"keys {SMALL_IDS[i]} fp8 kernel={kernel}")
    check_keys(orc, small_case(i), kernel, what=SMALL_IDS[i])


@pytest.mark.parametrize("kernel", [H16, H32, ROLES, H64, FP8, FP8_H32])
@pytest.mark.parametrize("keys", [16, 32, 48, 96, 160, 1024])
def test_keys_forced_splits(orc, keys, kernel):
    """Split boundaries at every forced size, on a C4 case with scattered
    unused entries (some splits hold only unused entries or only window keys)
    and a C128 case."""
    kv = "fp8" if kernel in FP8_KERNELS else "bf16"
    cases = [make_case(seq_lens=[3000, 700, 5], n_q=[2, 3, 1], H=100, R=4, seed=31, pad_mode="scatter", kv=kv,
                       n_sel=200),
             make_case(seq_lens=[9000, 130], n_q=[3, 1], H=64, R=128, seed=32, kv=kv)]
    for c in cases:
        log(f"keys forced split {keys} kernel={kernel} R={c.R}")
        check_keys(orc, c, kernel, split_keys=keys, what=f"R{c.R}-split{keys}-k{kernel}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_keys_workloads_default_plan(orc, n):
    """The five full-size workloads in the launch plan the benchmark times."""
    case = make_config(n)
    splits, chunk, kern = check_keys(orc, case, what=case.name)
    log(f"keys workload {n}: kernel {kern}, {splits} x {chunk} keys, all {case.T} rows bit-exact")


@pytest.mark.parametrize("kernel", [H16, H32, H64])
@pytest.mark.parametrize("n", [2, 3, 4])
def test_keys_workloads_other_kernels(orc, n, kernel):
    case = make_config(n)
    check_keys(orc, case, kernel, what=f"{case.name}-k{kernel}")


@pytest.mark.parametrize("kernel", [FP8, FP8_H32])
def test_keys_fp8_workload_both_kernels(orc, kernel):
    case = make_config(5)
    check_keys(orc, case, kernel, what=f"{case.name}-k{kernel}")


@pytest.mark.parametrize("kernel", [0, H16, H32, ROLES, H64])
@pytest.mark.parametrize("n", [6, 7])
def test_keys_prefill_reduced(orc, n, kernel):
    """Prefill rows (2 requests x 96 rows): every row's keys, bit-exact."""
    case = make_config(n, batch=2, rows=96)
    check_keys(orc, case, kernel, what=f"{case.name}-reduced-k{kernel}")


@pytest.mark.parametrize("kernel", [0, H16, H32, ROLES, H64, FP8, FP8_H32])
def test_keys_page_table_beyond_lds_cache(orc, kernel):
    """Requests whose extra page table is longer than a workgroup's LDS cache
    of it (contexts past 1M tokens): compressed slots resolved through one
    more round of page-table loads, bit-exact on every variant."""
    kv = "fp8" if kernel in FP8_KERNELS else "bf16"
    case = make_case(seq_lens=[1_200_000, 1_060_000], n_q=[1, 3], H=64, R=4, seed=91, kv=kv)
    assert case.extra_page_table.shape[1] > 1024
    log(f"keys beyond the page-table cache kernel={kernel}")
    check_keys(orc, case, kernel, what=f"beyond-cache-k{kernel}")


@pytest.mark.parametrize("kernel", [0, H16, H32, ROLES, H64, FP8, FP8_H32])
@pytest.mark.parametrize("R", [4, 128])
def test_keys_many_requests(orc, R, kernel):
    """150 requests: rows past the first 64-request chunk of the
    row-to-request search, bit-exact key sets on every variant."""
    kv = "fp8" if kernel in FP8_KERNELS else "bf16"
    rng = np.random.default_rng(500 + R)
    B = 150
    nq = rng.integers(0, 4, size=B)
    sl = np.maximum(rng.integers(1, 700, size=B), nq) + (128 if R == 128 else 0)
    case = make_case(seq_lens=sl, n_q=nq, H=64, R=R, seed=501 + R, kv=kv, n_sel=40)
    log(f"keys many requests R={R} kernel={kernel}")
    check_keys(orc, case, kernel, what=f"many-requests-R{R}-k{kernel}")
