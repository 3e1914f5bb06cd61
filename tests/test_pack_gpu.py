"""GPU parity of the FP8 KV store (dsv4_kv_pack_fp8) against the oracle's
packer: the pool bytes must be identical (every code is an integer decided
from the same fp32 quotient on both sides).  Also: the bench-size launch on
sampled rows, and the attention reading a pool written by the kernel."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as oracle_mod
from synth import make_case
from synth.workloads import FP8_PAGE_BYTES, _to_bf16_bits
from tests import gpu_util as G

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.Oracle()


def log(msg):
    print(msg, flush=True)


def _gpu_pack(k_bits, slots, pool):
    from hybrid_sparse_mqa_amd import dsv4_kv_pack_fp8

    k = torch.from_numpy(np.ascontiguousarray(k_bits).view(np.int16)).view(torch.bfloat16).cuda()
    s = torch.from_numpy(np.ascontiguousarray(slots, np.int32)).cuda()
    p = torch.from_numpy(np.ascontiguousarray(pool)).cuda()
    dsv4_kv_pack_fp8(k, s, p)
    torch.cuda.synchronize()
    return p.cpu().numpy()


def _varied_rows(rng, n):
    """Normal rows scaled per row over 1e-6 .. 1e3, some with one large entry."""
    k = rng.standard_normal((n, 512)).astype(np.float32)
    k *= np.exp(rng.uniform(np.log(1e-6), np.log(1e3), (n, 1))).astype(np.float32)
    spikes = rng.random(n) < 0.2
    k[spikes, rng.integers(0, 448, spikes.sum())] *= 500.0
    return _to_bf16_bits(k)


def _compare(orc, k_bits, slots, pages, what):
    init = np.full((pages, FP8_PAGE_BYTES), 0xA5, np.uint8)
    want = init.copy()
    orc.pack_fp8(k_bits, slots, want)
    got = _gpu_pack(k_bits, slots, init)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} bytes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("n", [1000, 16384 + 5])  # one row per wave; four per wave with a ragged tail
def test_pack_random_rows_bit_exact(orc, n):
    rng = np.random.default_rng(1)
    pages = (n + 255) // 256 + 1
    k = _varied_rows(rng, n)
    slots = rng.permutation(pages * 256)[:n].astype(np.int32)
    slots[rng.random(n) < 0.1] = -1                       # skipped rows leave the pool untouched
    log(f"pack: {n} rows into {pages} pages")
    _compare(orc, k, slots, pages, "random rows")


def test_pack_edge_rows_bit_exact(orc):
    v = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()  # finite, ascending
    mids = (v[:-1] + v[1:]) / 2                                   # exact ties (4 mantissa bits fit bf16)
    rows = []
    r = np.zeros(512, np.float32); r[:448] = np.resize(np.concatenate([mids, -mids]), 448); r[0] = 448.0
    rows.append(r)                                                # scale 1: every tie goes to the even code
    r = np.zeros(512, np.float32); r[:448] = np.resize(np.concatenate([v, -v]), 448); r[1] = 448.0
    rows.append(r)                                                # every finite value, subnormals included
    rows.append(np.zeros(512, np.float32))                        # zero row: scale 1
    r = np.full(512, -0.0, np.float32); r[448:] = 3.0
    rows.append(r)                                                # negative zeros
    r = np.full(512, 7.0, np.float32); rows.append(r)             # constant row: all top codes
    r = np.zeros(512, np.float32); r[:448] = 2.0 ** -12; r[7] = 1e4
    rows.append(r)                                                # tiny quotients under one huge entry
    r = np.zeros(512, np.float32); r[:448] = np.linspace(-1, 1, 448) * 3e38; rows.append(r)
    k = _to_bf16_bits(np.stack(rows))
    log(f"pack: {len(rows)} edge rows")
    _compare(orc, k, np.arange(len(rows), dtype=np.int32), 1, "edge rows")


def test_pack_bench_size_sampled(orc):
    """The launch the benchmark times (65536 rows into 256 pages), checked on
    a sample of rows (the oracle packs rows independently)."""
    rng = np.random.default_rng(2)
    pages, n = 256, 65536
    k = _varied_rows(rng, n)
    slots = rng.permutation(pages * 256).astype(np.int32)
    log(f"pack: {n} rows into {pages} pages (sampled check)")
    got = _gpu_pack(k, slots, np.zeros((pages, FP8_PAGE_BYTES), np.uint8))
    pick = rng.choice(n, 600, replace=False)
    want = np.zeros_like(got)
    orc.pack_fp8(k[pick], slots[pick], want)
    for i in pick:
        page, rec = divmod(int(slots[i]), 256)
        a = slice(rec * 576, rec * 576 + 576)
        sc = slice(256 * 576 + 4 * rec, 256 * 576 + 4 * rec + 4)
        assert np.array_equal(got[page, a], want[page, a]) and np.array_equal(got[page, sc], want[page, sc]), i


def test_attention_reads_what_the_kernel_packed(orc):
    """Every record of an FP8 case's pools rewritten by the kernel (and, on the
    host, by the oracle's packer): same bytes, and the attention over the
    kernel-written pools matches the oracle over the oracle-written ones."""
    case = make_case(seq_lens=[700, 1500], n_q=[1, 3], H=64, R=4, kv="fp8", seed=4)
    rng = np.random.default_rng(3)
    pools = {}
    for name in ("swa_pool", "extra_pool"):
        pool = getattr(case, name)
        n = pool.shape[0] * 256
        k = _to_bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))  # N(0, 1) keys, as the generator draws
        slots = np.arange(n, dtype=np.int32)
        want = pool.copy()
        orc.pack_fp8(k, slots, want)
        got = _gpu_pack(k, slots, pool)
        assert np.array_equal(got, want), name
        pools[name] = want
    case = dataclasses.replace(case, **pools)
    log("pack: attention over kernel-packed pools")
    out, lse = G.run_forward(case)
    ro, rl, _ = orc.attention(case)
    G.compare(out, lse, ro, rl, what="packed pools")
