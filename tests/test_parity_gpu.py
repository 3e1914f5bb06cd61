"""GPU parity of the HIP path against the fp64 oracle (run with -m gpu).

* gather stage: slot lists and counts bit-exact, every row, all workloads;
* attention: every row of small cases (page edges, window edges, verify,
  multi-request, ragged, H from 1 to 128, W 1/3/128, bf16 and FP8) and every
  row of the five full-size workloads in the benchmark's launch plan;
* invariants on the GPU: physical page permutation is bit-identical, forced
  split sizes agree, repeated calls are bit-identical;
* sink variants; spike tests at every visibility edge and at split
  boundaries, on every kernel variant including FP8; the full E4M3 code
  table; empty passes, strided tensors, validate mode, graph capture.
(The bit-exact key sets of the split kernels themselves: test_keys_gpu.py.)
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle as oracle_mod
from synth import make_case, make_config, tile_requests
from tests import gpu_util as G

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.Oracle()


def log(msg):
    print(msg, flush=True)


# --------------------------------------------------------------------------
# gather stage
# --------------------------------------------------------------------------
def check_gather(orc, case, rows=None):
    slots, counts = G.run_gather(case)
    rows = range(case.T) if rows is None else rows
    for t in rows:
        swa, ext = orc.gather(case, t)
        assert counts[t, 0] == len(swa) and counts[t, 1] == len(ext), (t, counts[t], len(swa), len(ext))
        ref = np.concatenate([swa, ext])
        assert np.array_equal(slots[t, : len(ref)], ref), t
        assert np.all(slots[t, len(ref):] == -1)


SMALL = [  # (seq_lens, n_q, R, W, H, kv, extra kwargs)
    ([200], 1, 0, 128, 8, "bf16", {}),
    ([255], 1, 0, 128, 64, "bf16", {}),
    ([256], 1, 0, 128, 64, "bf16", {}),
    ([257], 1, 0, 128, 64, "bf16", {}),
    ([128], 1, 0, 128, 64, "bf16", {}),
    ([260], 4, 0, 128, 64, "bf16", {}),
    ([256], 16, 0, 128, 16, "bf16", {}),
    ([32, 96], 1, 0, 128, 64, "bf16", {}),
    ([300, 5, 1], [3, 1, 1], 0, 3, 33, "bf16", {}),
    ([64], 1, 4, 128, 64, "bf16", {}),
    ([80], 16, 4, 128, 64, "bf16", {}),
    ([67, 99], 3, 4, 128, 64, "bf16", dict(pad_mode="scatter", n_sel=7)),
    ([3000, 700], [4, 2], 4, 128, 128, "bf16", dict(pad_mode="scatter")),
    ([128], 1, 128, 128, 64, "bf16", {}),
    ([144], 16, 128, 128, 64, "bf16", {}),
    ([131, 163, 2000], 3, 128, 128, 100, "bf16", {}),
    ([9000], 2, 128, 1, 1, "bf16", {}),
    ([5000, 12], [4, 0], 4, 128, 64, "fp8", {}),
    ([600, 90], [1, 3], 128, 128, 8, "fp8", {}),
    ([200], 1, 0, 128, 64, "fp8", {}),
    ([3000, 700, 5], [2, 3, 1], 4, 3, 128, "fp8", dict(pad_mode="scatter", n_sel=300)),
    ([131, 2000], [3, 1], 128, 128, 33, "fp8", {}),
]
SMALL_IDS = [f"{i}-R{c[2]}-W{c[3]}-H{c[4]}-{c[5]}" for i, c in enumerate(SMALL)]


def small_case(i, **over):
    sl, nq, R, W, H, kv, extra = SMALL[i]
    kw = dict(seq_lens=sl, n_q=nq, R=R, W=W, H=H, kv=kv, seed=500 + i, K=512 if R == 4 else 512)
    kw.update(extra)
    kw.update(over)
    return make_case(**kw)


@pytest.mark.parametrize("i", range(len(SMALL)), ids=SMALL_IDS)
def test_gather_small_bit_exact(orc, i):
    check_gather(orc, small_case(i))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_gather_workloads_bit_exact(orc, n):
    log(f"gather workload {n}")
    check_gather(orc, make_config(n))


# bf16 split-kernel variants (DSV4_KERNEL_*): 0 automatic, 1 16 heads, 2 32 heads
# (dim quarters), 3 32 heads (score / PV roles), 4 64 heads.
BF16_KERNELS = [1, 2, 3, 4]
# FP8 split-kernel variants: 5 64 heads (dim halves), 6 32 heads (dim quarters).
FP8_KERNELS = [5, 6]


@pytest.fixture
def kernel(request):
    """Force one kernel variant for the test (it applies to pools of its own
    format), then restore the automatic choice."""
    from hybrid_sparse_mqa_amd import dsv4_attn_set_kernel

    dsv4_attn_set_kernel(request.param)
    yield request.param
    dsv4_attn_set_kernel(0)


def widen_extra_table(case, pages):
    """Pad each request's extra page-table row to `pages` columns with the
    poison page: the keys do not change, but the row no longer fits the
    split kernels' LDS copy of the table (1024 pages)."""
    et = case.extra_page_table
    wide = np.full((et.shape[0], pages), case.poison_extra_page, dtype=np.int32)
    wide[:, : et.shape[1]] = et
    return dataclasses.replace(case, extra_page_table=wide)


@pytest.mark.parametrize("kernel", [0] + BF16_KERNELS, indirect=True)
@pytest.mark.parametrize("i", [9, 12, 14, 17])
def test_extra_table_wider_than_lds_copy(orc, i, kernel):
    case = widen_extra_table(small_case(i), 1100)
    log(f"wide extra table {SMALL_IDS[i]} kernel={kernel}")
    check_gather(orc, case)
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"wide-{SMALL_IDS[i]}-k{kernel}")


# --------------------------------------------------------------------------
# attention, small cases, every row
# --------------------------------------------------------------------------
@pytest.mark.parametrize("i", range(len(SMALL)), ids=SMALL_IDS)
def test_forward_small(orc, i):
    case = small_case(i)
    log(f"forward small {SMALL_IDS[i]} T={case.T}")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=SMALL_IDS[i])


@pytest.mark.parametrize("kernel", BF16_KERNELS, indirect=True)
@pytest.mark.parametrize("i", [0, 3, 5, 8, 11, 12, 14, 15, 16], ids=[SMALL_IDS[i] for i in [0, 3, 5, 8, 11, 12, 14, 15, 16]])
def test_forward_small_each_bf16_kernel(orc, i, kernel):
    case = small_case(i)
    log(f"forward small {SMALL_IDS[i]} kernel={kernel}")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"{SMALL_IDS[i]}-k{kernel}")


FP8_SMALL = [i for i, c in enumerate(SMALL) if c[5] == "fp8"]


@pytest.mark.parametrize("kernel", FP8_KERNELS, indirect=True)
@pytest.mark.parametrize("i", FP8_SMALL, ids=[SMALL_IDS[i] for i in FP8_SMALL])
def test_forward_small_each_fp8_kernel(orc, i, kernel):
    case = small_case(i)
    log(f"forward small {SMALL_IDS[i]} kernel={kernel}")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"{SMALL_IDS[i]}-k{kernel}")


@pytest.mark.parametrize("kernel", BF16_KERNELS, indirect=True)
@pytest.mark.parametrize("keys", [16, 32, 48, 96, 160, 2048])
def test_forced_split_sizes_each_bf16_kernel(orc, keys, kernel):
    from hybrid_sparse_mqa_amd import dsv4_attn_set_split_keys

    case = make_case(seq_lens=[3000, 700, 5], n_q=[2, 3, 1], H=100, R=4, seed=31, pad_mode="scatter")
    ro, rl, _ = orc.attention(case)
    dsv4_attn_set_split_keys(keys)
    try:
        out, lse = G.run_forward(case)
    finally:
        dsv4_attn_set_split_keys(0)
    G.compare(out, lse, ro, rl, what=f"split{keys}-k{kernel}")


def _random_wide_case(seed):
    """Random shapes that reach the planner's other branches: many requests
    (grids past one round of workgroups, where the 64-head kernels take
    over), long C128 rows (more keys than one workgroup's limit: equal
    splits), and small mixed cases."""
    rng = np.random.default_rng(seed)
    R = int(rng.choice([0, 4, 128]))
    mode = rng.random()
    if mode < 0.3:
        B = int(rng.integers(64, 300))
        nq = rng.integers(1, 3, size=B)
        sl = np.maximum(rng.integers(1, 3000, size=B), nq)
    elif mode < 0.7 and R == 128:
        B = int(rng.integers(1, 4))
        nq = rng.integers(1, 4, size=B)
        sl = rng.integers(100_000, 200_000, size=B)
    else:
        B = int(rng.integers(1, 9))
        nq = rng.integers(0, 6, size=B)
        sl = np.maximum(rng.integers(1, 6000, size=B), nq) + (int(rng.integers(0, 300)) if R == 128 else 0)
    heads = [16, 33, 64] if mode < 0.3 else [1, 5, 16, 17, 32, 33, 64, 65, 100, 128]
    case = make_case(seq_lens=sl, n_q=nq, H=int(rng.choice(heads)), R=R, W=int(rng.choice([1, 2, 3, 64, 128, 200])),
                     kv=str(rng.choice(["bf16", "fp8"])), sink=bool(rng.random() < 0.8), seed=9000 + seed,
                     K=int(rng.choice([32, 64, 512, 600])), pad_mode=str(rng.choice(["tail", "scatter"])))
    return case, int(rng.choice([0, 0, 32, 64, 96, 160]))


@pytest.mark.parametrize("seed", range(2000, 2040))
def test_forward_random_every_variant(orc, seed):
    """Random cases (see _random_wide_case) on the automatic plan and every
    variant of the pool's format, under a random forced split size."""
    from hybrid_sparse_mqa_amd import dsv4_attn_set_kernel, dsv4_attn_set_split_keys

    case, split = _random_wide_case(seed)
    if case.T == 0:
        pytest.skip("no query rows drawn")
    log(f"random every variant seed={seed} R={case.R} T={case.T} H={case.H} W={case.W} kv={case.kv} split={split}")
    ro, rl, _ = orc.attention(case)
    for k in ([0] + FP8_KERNELS if case.kv == "fp8" else [0] + BF16_KERNELS):
        dsv4_attn_set_kernel(k)
        dsv4_attn_set_split_keys(split)
        try:
            out, lse = G.run_forward(case)
        finally:
            dsv4_attn_set_kernel(0)
            dsv4_attn_set_split_keys(0)
        G.compare(out, lse, ro, rl, what=f"random seed {seed} k{k} split{split}")


@pytest.mark.parametrize("seed", range(6))
def test_forward_random(orc, seed):
    rng = np.random.default_rng(seed)
    R = int(rng.choice([0, 4, 128]))
    B = int(rng.integers(1, 5))
    nq = rng.integers(0, 5, size=B)
    sl = np.maximum(rng.integers(1, 4000, size=B), nq)
    if R == 128:
        sl = sl + 128
    case = make_case(seq_lens=sl, n_q=nq, H=int(rng.choice([1, 7, 32, 64, 65, 128])), R=R,
                     W=int(rng.choice([1, 3, 128, 200])), kv=str(rng.choice(["bf16", "fp8"])),
                     sink=bool(rng.random() < 0.8), seed=700 + seed,
                     K=int(rng.choice([64, 512, 600])), pad_mode=str(rng.choice(["tail", "scatter"])))
    log(f"forward random seed={seed} R={R} T={case.T} H={case.H} W={case.W} kv={case.kv}")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"random {seed}")


# --------------------------------------------------------------------------
# full-size workloads, benchmark launch plan, sampled rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_forward_workloads_all_rows(orc, n):
    """The five full-size workloads in the benchmark's launch plan, every row
    against the oracle."""
    case = make_config(n)
    log(f"forward workload {n} ({case.name}) all {case.T} rows")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    e = G.compare(out, lse, ro, rl, what=case.name)
    log(f"  max abs err {e[0]:.3g}  lse err {e[1]:.3g}  rel L2 {e[2]:.3g}")


@pytest.mark.parametrize("kernel", FP8_KERNELS, indirect=True)
def test_forward_fp8_1m_tiled_batch_all_rows(orc, kernel):
    """The FP8 1M-token decode at a larger batch, built as the benchmark's
    batch sweep builds it (copies of two requests, each copy through its own
    C4 lists): 32 rows, every row against the oracle."""
    case = tile_requests(make_config(5, batch=2, index_sets=16), 16)
    log(f"forward {case.name} tiled to {case.B} requests")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    e = G.compare(out, lse, ro, rl, what="fp8-1m-tiled")
    log(f"  max abs err {e[0]:.3g}  lse err {e[1]:.3g}  rel L2 {e[2]:.3g}")


# --------------------------------------------------------------------------
# invariants on the GPU
# --------------------------------------------------------------------------
def permute_pages(case, seed):
    rng = np.random.default_rng(seed)
    fp8 = case.kv == "fp8"

    def perm(pool, table):
        n = pool.shape[0] if fp8 else pool.shape[0] // 256
        pi = rng.permutation(n)
        pages = pool if fp8 else pool.reshape(n, 256, 512)
        new = np.empty_like(pages)
        new[pi] = pages
        return (new if fp8 else new.reshape(-1, 512)), pi[table].astype(np.int32)

    swa, st = perm(case.swa_pool, case.swa_page_table)
    ext, et = case.extra_pool, case.extra_page_table
    if ext is not None:
        ext, et = perm(ext, et)
    return dataclasses.replace(case, swa_pool=swa, swa_page_table=st, extra_pool=ext, extra_page_table=et)


@pytest.mark.parametrize("i", [5, 12, 15, 18])
def test_page_permutation_bit_identical(i):
    case = small_case(i)
    a_out, a_lse = G.run_forward(case)
    b_out, b_lse = G.run_forward(permute_pages(case, 99))
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


def test_repeat_bit_identical():
    case = small_case(12)
    g = G.to_gpu(case)
    a = G.run_forward(case, g)
    b = G.run_forward(case, g)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("keys", [32, 64, 96, 160, 256, 1024])
def test_forced_split_sizes(orc, keys):
    from hybrid_sparse_mqa_amd import dsv4_attn_set_split_keys

    case = small_case(12)
    ro, rl, _ = orc.attention(case)
    try:
        dsv4_attn_set_split_keys(keys)
        out, lse = G.run_forward(case)
    finally:
        dsv4_attn_set_split_keys(0)
    G.compare(out, lse, ro, rl, what=f"split {keys}")


# --------------------------------------------------------------------------
# sink variants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["none", "-1e30", "zero", "normal", "+30"])
def test_sink_variants(orc, variant):
    kw = {}
    if variant == "none":
        kw = dict(sink=False)
    elif variant == "normal":
        kw = dict(sink=True)
    else:
        kw = dict(sink=True, sink_value={"-1e30": -1e30, "zero": 0.0, "+30": 30.0}[variant])
    case = make_case(seq_lens=[700, 300], n_q=[2, 1], H=64, R=128, seed=31, **kw)
    out, lse = G.run_forward(case)
    ro, rl, rns = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"sink {variant}")
    if variant in ("none", "-1e30"):
        assert np.allclose(lse.cpu().numpy(), rns, atol=G.LSE_ATOL, rtol=0)


# --------------------------------------------------------------------------
# spike tests: a key pointing along q[t, 0] must dominate head 0 exactly when
# it is visible to the row
# --------------------------------------------------------------------------
SPIKES = [
    # (name, R, seq_lens, n_q, where, visible)
    ("window first", 0, [1000], 1, "tok:p-W+1", True),
    ("window before", 0, [1000], 1, "tok:p-W", False),
    ("verify next row", 0, [1000], 4, "tok:p+1", False),
    ("c128 last visible", 128, [1026], 4, "cmp:vis-1", True),
    ("c128 first hidden", 128, [1026], 4, "cmp:vis", False),
    ("c4 listed", 4, [3000], 2, "c4:listed", True),
    ("c4 last used entry", 4, [3000], 2, "c4:last", True),
    ("c4 unlisted", 4, [3000], 2, "c4:unlisted", False),
]
# (kernel forced, kv): every bf16 variant, the automatic choice, and both FP8 variants.
VARIANTS = [(0, "bf16"), (1, "bf16"), (2, "bf16"), (3, "bf16"), (4, "bf16"), (5, "fp8"), (6, "fp8")]
VARIANT_IDS = ["auto", "h16", "h32", "roles", "h64", "fp8", "fp8-h32"]


@pytest.fixture
def variant(request):
    from hybrid_sparse_mqa_amd import dsv4_attn_set_kernel

    k, kv = request.param
    dsv4_attn_set_kernel(k)
    yield k, kv
    dsv4_attn_set_kernel(0)


def _slot(table, r, x):
    return int(table[r, x // 256]) * 256 + x % 256


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS, indirect=True)
@pytest.mark.parametrize("R", [0, 4, 128])
def test_many_requests(orc, R, variant):
    """150 requests (more than one 64-request chunk of the row-to-request
    search), decode and verify rows of ragged lengths, some requests without
    rows; every row checked on every kernel variant."""
    _, kv = variant
    rng = np.random.default_rng(500 + R)
    B = 150
    nq = rng.integers(0, 4, size=B)
    sl = np.maximum(rng.integers(1, 700, size=B), nq) + (128 if R == 128 else 0)
    case = make_case(seq_lens=sl, n_q=nq, H=64, R=R, seed=501 + R, kv=kv, n_sel=40)
    log(f"many requests B={B} T={case.T} R={R} kv={kv}")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"many requests R{R} {kv}")


_BEYOND_CACHE = {}


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS, indirect=True)
def test_page_table_beyond_lds_cache(orc, variant):
    """C4 rows of requests whose extra page table has more entries than a
    workgroup caches in LDS (1024 pages, i.e. contexts past 1M tokens): the
    split kernels resolve compressed slots through one more round of
    page-table loads.  A decode row and three verify rows; every row
    checked, on every kernel variant."""
    _, kv = variant
    if kv not in _BEYOND_CACHE:
        _BEYOND_CACHE.clear()  # one case on the device at a time
        case = make_case(seq_lens=[1_200_000, 1_060_000], n_q=[1, 3], H=64, R=4, seed=91, kv=kv)
        _BEYOND_CACHE[kv] = (case, G.to_gpu(case), orc.attention(case))
    case, g, (ro, rl, _) = _BEYOND_CACHE[kv]
    assert case.extra_page_table.shape[1] > 1024
    log(f"page table beyond the LDS cache: {case.extra_page_table.shape[1]} pages, kv={kv}")
    out, lse = G.run_forward(case, g)
    G.compare(out, lse, ro, rl, what=f"table beyond cache {kv}")


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS, indirect=True)
@pytest.mark.parametrize("name,R,sl,nq,where,visible", SPIKES, ids=[s[0] for s in SPIKES])
def test_spikes(orc, name, R, sl, nq, where, visible, variant):
    _, kv = variant
    case = make_case(seq_lens=sl, n_q=nq, H=64, R=R, seed=77, n_sel=300, kv=kv)
    t = 0  # first row of the request
    p = int(case.seq_lens[0]) - nq + 0
    kind, pos = where.split(":")
    if kind == "tok":
        x = {"p-W+1": p - case.W + 1, "p-W": p - case.W, "p+1": p + 1}[pos]
        G.spike_slot(case, "swa_pool", _slot(case.swa_page_table, 0, x), t)
    elif kind == "cmp":
        vis = (p + 1) // 128
        x = vis - 1 if pos == "vis-1" else vis
        assert x < int(case.seq_lens[0]) // 128
        G.spike_slot(case, "extra_pool", _slot(case.extra_page_table, 0, x), t)
    else:
        listed = case.c4_indices[t][case.c4_indices[t] >= 0]
        if pos == "listed":
            x = int(listed[17])
        elif pos == "last":
            x = int(listed[-1])  # index n_sel - 1 of the list, followed by -1 padding
            assert case.c4_indices[t][len(listed)] == -1
        else:
            vis = (p + 1) // 4
            x = int(np.setdiff1d(np.arange(vis), listed)[3])
        G.spike_slot(case, "extra_pool", _slot(case.extra_page_table, 0, x), t)
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=name)
    dominated = rl[t, 0] > 50.0
    assert dominated == visible, (name, rl[t, 0])


@pytest.mark.parametrize("variant", VARIANTS[1:], ids=VARIANT_IDS[1:], indirect=True)
@pytest.mark.parametrize("R", [4, 128])
@pytest.mark.parametrize("keys", [32, 64, 96])
def test_spikes_at_split_boundaries(orc, keys, R, variant):
    """Under forced split sizes, a spike on the first and on the last key of
    a split (in the kernel's own key order), and on the row's last key, must
    each dominate: no split boundary drops or duplicates a key."""
    from hybrid_sparse_mqa_amd import dsv4_attn_set_split_keys

    kernel, kv = variant
    compressed_first = kernel in (2, 3, 4)
    base = dict(seq_lens=[2600], n_q=2, H=64, R=R, seed=88, kv=kv, n_sel=200, pad_mode="scatter")
    probe = make_case(**base)
    t = 1
    order = G.expected_keys(orc, probe, t, compressed_first)
    n = len(order)
    chunk = -(-keys // (16 if kernel == 1 else 32)) * (16 if kernel == 1 else 32)
    where = sorted({i for i in (chunk - 1, chunk, 2 * chunk - 1, 2 * chunk, 3 * chunk - 1, n - 1) if 0 <= i < n})
    dsv4_attn_set_split_keys(keys)
    try:
        for i in where:
            if order[i] is None:  # an unused C4 entry: the nearest used key before it
                i = max(j for j in range(i) if order[j] is not None)
            case = make_case(**base)
            pool, slot = order[i]
            G.spike_slot(case, "swa_pool" if pool == "swa" else "extra_pool", slot, t)
            out, lse = G.run_forward(case)
            ro, rl, _ = orc.attention(case)
            G.compare(out, lse, ro, rl, what=f"boundary key {i} split {keys} R{R} k{kernel} {kv}")
            assert rl[t, 0] > 50.0, (i, rl[t, 0])
    finally:
        dsv4_attn_set_split_keys(0)


@pytest.mark.parametrize("kernel", FP8_KERNELS, indirect=True)
@pytest.mark.parametrize("R", [0, 128])
def test_growing_scores_fp8(orc, R, kernel):
    """The growing-score test on packed FP8 pools: every key row of row 0 is
    re-stored (quantised) as the blend towards 2 * q[0, head 0]."""
    from synth import store_float_rows

    case = make_case(seq_lens=[40000, 300], n_q=[1, 2], H=64, R=R, seed=54, kv="fp8")
    q0 = torch.from_numpy(case.q[0, 0].view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    swa, ext = orc.gather(case, 0)
    n = len(swa) + len(ext)
    rng = np.random.default_rng(9)
    for pool_name, slots, base in (("swa_pool", swa, 0), ("extra_pool", ext, len(swa))):
        beta = (base + np.arange(len(slots))) / max(n - 1, 1)
        rows = (1.0 - beta)[:, None] * rng.standard_normal((len(slots), 512)) + beta[:, None] * 2.0 * q0[None, :]
        store_float_rows(getattr(case, pool_name), "fp8", slots, rows.astype(np.float32))
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"growing-fp8-R{R}-k{kernel}")


@pytest.mark.parametrize("kernel", FP8_KERNELS, indirect=True)
@pytest.mark.parametrize("keys", [32, 64, 160, 1024])
def test_forced_split_sizes_fp8(orc, keys, kernel):
    from hybrid_sparse_mqa_amd import dsv4_attn_set_split_keys

    case = make_case(seq_lens=[3000, 700, 5], n_q=[2, 3, 1], H=100, R=4, seed=31, pad_mode="scatter", kv="fp8")
    ro, rl, _ = orc.attention(case)
    dsv4_attn_set_split_keys(keys)
    try:
        out, lse = G.run_forward(case)
    finally:
        dsv4_attn_set_split_keys(0)
    G.compare(out, lse, ro, rl, what=f"fp8 split{keys} k{kernel}")


@pytest.mark.parametrize("kernel", BF16_KERNELS, indirect=True)
@pytest.mark.parametrize("R", [0, 128])
def test_growing_scores(orc, R, kernel):
    """Key rows of row 0 blend, along its key list, from random towards
    2 * q[0, head 0], so head 0's scores climb by about 65 (base 2) over the
    pass: its running softmax reference falls far behind later keys several
    times (for the 16-head kernel, a restart of the wave's tiles each time),
    while the values stay near unit scale."""
    case = make_case(seq_lens=[40000, 300], n_q=[1, 2], H=64, R=R, seed=53)
    q0 = torch.from_numpy(case.q[0, 0].view(np.int16)).view(torch.bfloat16).float()
    swa, ext = orc.gather(case, 0)
    n = len(swa) + len(ext)
    for pool_name, slots, base in (("swa_pool", swa, 0), ("extra_pool", ext, len(swa))):
        pool = getattr(case, pool_name)
        for i, slot in enumerate(slots):
            beta = (base + i) / max(n - 1, 1)
            row = torch.from_numpy(pool[slot].view(np.int16)).view(torch.bfloat16).float()
            grown = ((1.0 - beta) * row + beta * 2.0 * q0).to(torch.bfloat16)
            pool[slot] = grown.view(torch.int16).numpy().view(np.uint16)
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"growing-R{R}-k{kernel}")


# --------------------------------------------------------------------------
# FP8: every finite E4M3 code through the dequant path
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", FP8_KERNELS, indirect=True)
def test_fp8_all_codes(orc, kernel):
    from synth.workloads import FP8_SCALE_OFFSET

    case = make_case(seq_lens=[2000], n_q=2, H=64, R=128, kv="fp8", seed=3)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for pool in (case.swa_pool, case.extra_pool):
        n_pages = pool.shape[0]
        rec = pool[:, :FP8_SCALE_OFFSET].reshape(n_pages, 256, 576)
        fill = np.resize(codes, (n_pages, 256, 448))  # every record cycles through all 254 codes
        live =~np.all(rec[:, :, :448] == 0xFF, axis=2)  # poisoned records stay poisoned
        rec[:, :, :448] = np.where(live[:, :, None], fill, rec[:, :, :448])
        pool[:, :FP8_SCALE_OFFSET] = rec.reshape(n_pages, -1)
        sc = np.full((n_pages, 256), 1.0 / 64, np.float32)
        old = pool[:, FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 1024].copy().view(np.float32)
        sc = np.where(np.isnan(old), old, sc)
        pool[:, FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 1024] = sc.view(np.uint8)
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what="fp8 codes")


def _fp8_pool_from_bf16(pool):
    """The packed FP8 pool holding the same rows as a bf16 pool (synth's
    quantiser: per-token scale amax/448, E4M3 codes, bf16 rotary dims);
    unbacked (poisoned) rows stay poisoned."""
    from synth.workloads import FP8_PAGE_BYTES, POISON_BYTE, store_float_rows

    pages = pool.shape[0] // 256
    out = np.full((pages, FP8_PAGE_BYTES), POISON_BYTE, dtype=np.uint8)
    live = np.nonzero(~np.all(pool == 0xFFFF, axis=1))[0]
    rows = (pool[live].astype(np.uint32) << 16).view(np.float32)
    store_float_rows(out, "fp8", live, rows)
    return out


@pytest.mark.parametrize("kernel", FP8_KERNELS, indirect=True)
@pytest.mark.parametrize("R", [4, 128])
def test_fp8_against_unquantised_bf16(orc, R, kernel):
    """How far FP8 storage moves the result (informational, bounded at the
    5e-2 with which the test-matrix page's reference notes absorb FP8 noise
    against the saved bf16 keys): the FP8 path over pools packed from a bf16
    case's rows, against the oracle on the unquantised bf16 rows."""
    base = make_case(seq_lens=[3000, 9000], n_q=[1, 2], H=64, R=R, seed=77)
    fp8 = dataclasses.replace(base, kv="fp8", swa_pool=_fp8_pool_from_bf16(base.swa_pool),
                              extra_pool=_fp8_pool_from_bf16(base.extra_pool))
    out, lse = G.run_forward(fp8)
    ro, rl, _ = orc.attention(base)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    err = np.abs(o - ro).max()
    rel = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    log(f"FP8 vs unquantised bf16 (R={R}): max abs {err:.3g}, rel L2 {rel:.3g}, lse {np.abs(l - rl).max():.3g}")
    assert np.allclose(o, ro, atol=5e-2, rtol=5e-2) and np.allclose(l, rl, atol=5e-2)


@pytest.mark.parametrize("kernel", FP8_KERNELS, indirect=True)
def test_fp8_decode_bit_exact(orc, kernel):
    """One visible key (position 0, window only), no sink, per-token scale 1:
    every head's softmax weight is exactly 1, so every output row is the key's
    dequantised row.  Its 448 codes cycle through all 254 finite E4M3 codes
    (subnormals and both zeros included), each of which is exact in bf16, so
    the output must equal the oracle's value exactly, not within tolerance."""
    from synth.workloads import FP8_ROW_BYTES, FP8_SCALE_OFFSET

    case = make_case(seq_lens=[1], n_q=1, H=64, R=0, kv="fp8", sink=False, seed=5)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    page = int(case.swa_page_table[0, 0])
    rec = 0  # position 0 is record 0 of the request's first page
    base = rec * FP8_ROW_BYTES
    case.swa_pool[page, base:base + 448] = np.resize(codes, 448)
    case.swa_pool[page, FP8_SCALE_OFFSET + 4 * rec:FP8_SCALE_OFFSET + 4 * rec + 4] = \
        np.array([1.0], np.float32).view(np.uint8)
    out, _ = G.run_forward(case)
    ro, _, _ = orc.attention(case)
    got = out.float().cpu().numpy()
    want = torch.from_numpy(ro.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(want, ro.astype(np.float32)), "the expected rows are not bf16-exact"
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} values differ, first at {bad[:4].tolist()}"


# --------------------------------------------------------------------------
# shapes and modes
# --------------------------------------------------------------------------
def test_empty_pass():
    case = make_case(seq_lens=[10, 20], n_q=[0, 0], H=8, R=0, seed=1)
    out, lse = G.run_forward(case)
    assert out.shape == (0, 8, 512) and lse.shape == (0, 8)


def test_without_lse_and_strided(orc):
    case = small_case(12)
    g = G.to_gpu(case)
    big_q = torch.zeros((case.T, case.H + 3, 520), dtype=torch.bfloat16, device="cuda")
    big_q[:, 1:case.H + 1, :512] = g["q"]
    g["q"] = big_q[:, 1:case.H + 1, :512]
    out_big = torch.full((case.T, case.H, 520), 7.0, dtype=torch.bfloat16, device="cuda")
    out, lse = G.run_forward(case, g, out=out_big[:, :, :512], return_lse=False)
    assert lse is None
    assert torch.all(out_big[:, :, 512:] == 7.0)
    ro, rl, _ = orc.attention(case)
    ref_out, ref_lse = G.run_forward(case)
    assert torch.equal(out_big[:, :, :512], ref_out)


def test_validate_mode_rejects_bad_index(monkeypatch):
    from hybrid_sparse_mqa_amd import Dsv4Error

    case = make_case(seq_lens=[300], n_q=1, H=8, R=4, seed=1, n_sel=4)
    case.c4_indices[0, 1] = 10 ** 6
    monkeypatch.setenv("DSV4_VALIDATE", "1")
    with pytest.raises(Dsv4Error, match="ERR_CONTRACT"):
        G.run_forward(case)


# --------------------------------------------------------------------------
# interleaved plans, workspace growth and graph capture
# --------------------------------------------------------------------------
def test_interleaved_calls_bit_identical():
    """Alternating cases with different split plans (and so different
    workspace layouts) stay bit-identical to their first results."""
    from hybrid_sparse_mqa_amd import dsv4_attn_set_split_keys

    cases = [small_case(12), small_case(15), make_case(seq_lens=[2000] * 9, n_q=1, H=64, R=128, seed=4)]
    gs = [G.to_gpu(c) for c in cases]
    first = [G.run_forward(c, g) for c, g in zip(cases, gs)]
    for rep in range(3):
        for keys in (0, 64, 0):
            try:
                dsv4_attn_set_split_keys(keys)
                for c, g, ref in zip(cases, gs, first):
                    out, lse = G.run_forward(c, g)
                    if keys == 0:
                        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
            finally:
                dsv4_attn_set_split_keys(0)


def test_reserve_then_capture_first_forward():
    """After releasing the workspace, a reserve followed by a capture whose
    forward is the first call since then works and replays correctly; without
    the reserve the captured call refuses to allocate (DSV4_ERR_WORKSPACE)
    instead of breaking the capture."""
    from hybrid_sparse_mqa_amd import (Dsv4Error, dsv4_attn_forward, dsv4_attn_plan, dsv4_attn_workspace_release,
                                       dsv4_attn_workspace_reserve)

    case = make_case(seq_lens=[3000, 5000, 700], n_q=[1, 4, 2], H=64, R=4, seed=14)
    g = G.to_gpu(case)
    splits, _, _ = dsv4_attn_plan(case.T, case.H, case.R, case.W, case.K, case.extra_page_table.shape[1])
    assert splits > 1  # the call needs the workspace
    ref_out, ref_lse = G.run_forward(case, g)

    def call(out, lse):
        dsv4_attn_forward(g["q"], g["swa_pool"], g["swa_page_table"], g["extra_pool"], g["extra_page_table"],
                          g["c4_indices"], g["seq_lens"], g["qo_indptr"], g["sink"], case.R, case.W, case.scale,
                          out=out, lse=lse)

    out = torch.zeros_like(ref_out)
    lse = torch.zeros_like(ref_lse)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    dsv4_attn_workspace_release()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(Dsv4Error, match="ERR_WORKSPACE"):
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                call(out, lse)
    torch.cuda.synchronize()
    dsv4_attn_workspace_reserve(case.T * splits * case.H * 1028, stream.cuda_stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            call(out, lse)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), rep
        G.run_forward(make_case(seq_lens=[9000] * 40, n_q=1, H=64, R=128, seed=4))  # grows the workspace
    # The buffer the graph captured is kept after growth: replays stay correct.
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_graph_capture_replays_match_eager():
    """A captured forward replays correctly several times, with eager calls
    (and synchronisations) in between."""
    from hybrid_sparse_mqa_amd import dsv4_attn_forward

    case = make_case(seq_lens=[3000, 5000, 700], n_q=[1, 4, 2], H=64, R=4, seed=12)
    g = G.to_gpu(case)
    ref_out, ref_lse = G.run_forward(case, g)
    out = torch.zeros_like(ref_out)
    lse = torch.zeros_like(ref_lse)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            dsv4_attn_forward(g["q"], g["swa_pool"], g["swa_page_table"], g["extra_pool"], g["extra_page_table"],
                              g["c4_indices"], g["seq_lens"], g["qo_indptr"], g["sink"], case.R, case.W, case.scale,
                              out=out, lse=lse)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), rep
        other = G.run_forward(small_case(12))  # eager work between replays
        assert torch.isfinite(other[0].float()).all()


@pytest.mark.gpu
def test_timing_events_eager_and_captured():
    """Kernel timing: eager calls on the null stream and on a side stream, and
    calls captured into a graph (event nodes re-recorded by each replay)."""
    from hybrid_sparse_mqa_amd import dsv4_attn_forward, dsv4_attn_timing_enable, dsv4_attn_timing_read

    case = make_case(seq_lens=[3000, 5000], n_q=[1, 2], H=64, R=4, seed=13)
    g = G.to_gpu(case)
    ref_out, ref_lse = G.run_forward(case, g)

    def call(out=None, lse=None):
        return dsv4_attn_forward(g["q"], g["swa_pool"], g["swa_page_table"], g["extra_pool"], g["extra_page_table"],
                                 g["c4_indices"], g["seq_lens"], g["qo_indptr"], g["sink"], case.R, case.W,
                                 case.scale, out=out, lse=lse)

    dsv4_attn_timing_read()  # clear
    dsv4_attn_timing_enable(True)
    try:
        # Eager calls: the kernels are launched with dispatch-attached events.
        for _ in range(2):
            o, l = call()
            torch.cuda.synchronize()
            assert torch.equal(o, ref_out) and torch.equal(l, ref_lse)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            o, l = call()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_out) and torch.equal(l, ref_lse)
        split_ms, merge_ms, n = dsv4_attn_timing_read()
        assert n == 3 and split_ms > 0 and merge_ms > 0  # this case splits its rows

        out = torch.zeros_like(ref_out)
        lse = torch.zeros_like(ref_lse)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                call(out, lse)
                call(out, lse)
    finally:
        dsv4_attn_timing_enable(False)
    torch.cuda.synchronize()
    for rep in range(2):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), rep
        split_ms, merge_ms, n = dsv4_attn_timing_read() if rep == 1 else (1.0, 0.0, 2)
        assert n == 2 and split_ms > 0 and merge_ms >= 0
    assert dsv4_attn_timing_read()[2] == 0


# --------------------------------------------------------------------------
# sparse prefill / extend: many query rows per request, each with its own
# causal window and (C4) its own top-512 list
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [6, 7])
def test_prefill_workloads_sampled_rows(orc, n):
    """The two full-size prefill workloads (4 requests x 2048 rows) in the
    benchmark's launch plan: the first and last rows of every request and 120
    random ones against the oracle."""
    case = make_config(n)
    rng = np.random.default_rng(n)
    ends = [int(x) for r in range(case.B) for x in (case.qo_indptr[r], case.qo_indptr[r + 1] - 1)]
    rows = sorted(set(ends + list(rng.choice(case.T, size=120, replace=False))))
    log(f"prefill workload {n} ({case.name}) {len(rows)} rows of {case.T}")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case, rows=rows)
    e = G.compare(out, lse, ro, rl, rows=rows, what=case.name)
    log(f"  max abs err {e[0]:.3g}  lse err {e[1]:.3g}  rel L2 {e[2]:.3g}")


@pytest.mark.parametrize("kernel", [0] + BF16_KERNELS, indirect=True)
@pytest.mark.parametrize("n", [6, 7])
def test_prefill_reduced_all_rows(orc, n, kernel):
    """The prefill shapes at 2 requests x 192 rows (a ragged 192 = 1.5 x 128
    rows, window edges inside the pass), every row, every bf16 variant."""
    case = make_config(n, batch=2, rows=192)
    log(f"prefill reduced {n} kernel={kernel} T={case.T}")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what=f"{case.name}-reduced-k{kernel}")
