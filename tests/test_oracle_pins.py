"""Pins of the fp64 oracle to things other than itself (CPU only).

* brute force over unpaged logical rows (tests/bruteforce.py), random tiny cases;
* closed forms (single key; N identical keys);
* invariants (physical page permutation, request permutation, sink -> -inf,
  C4 with no indices, C128 before the first complete block, SWA-only within
  the window == full causal attention, FP8 with exactly representable values
  == bf16);
* library routines (torch's bf16 and float8_e4m3fn tables);
* the integer worked examples printed by the DSV4 walk-through page;
* mutants: deliberately wrong builds of the oracle must fail at least one pin.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle as oracle_mod
from synth import make_case
from tests import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


@pytest.fixture(scope="module")
def orc():
    oracle_mod.build()
    return oracle_mod.Oracle()


def _close(a, b, tol=TOL):
    a = np.asarray(a)
    b = np.asarray(b)
    return a.shape == b.shape and np.all(np.isfinite(a)) and np.allclose(a, b, rtol=tol, atol=tol)


# --------------------------------------------------------------------------
# storage decoding against library tables
# --------------------------------------------------------------------------
def test_e4m3fn_table_matches_torch(orc):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_to_double(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def test_bf16_all_patterns_match_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bruteforce.bf16_bits_to_f64(bits)
    got = np.array([orc.bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(ref[~np.isnan(ref)], got[~np.isnan(got)])
    # bit patterns, so that +0/-0 and the infinities are told apart too
    ok = ~np.isnan(ref)
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------
def _random_case(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.choice([0, 4, 128]))
    W = int(rng.choice([1, 3, 128]))
    B = int(rng.integers(1, 4))
    nq = rng.integers(1, 5, size=B)
    lo = 1 if R != 128 else 100
    sl = np.maximum(rng.integers(lo, 600, size=B), nq)
    kv = "fp8" if rng.random() < 0.35 else "bf16"
    return make_case(seq_lens=sl, n_q=nq, H=int(rng.integers(1, 5)), R=R, W=W, kv=kv,
                     sink=bool(rng.random() < 0.8), seed=seed, keep_logical=True,
                     n_sel=int(rng.integers(1, 60)), pad_mode=str(rng.choice(["tail", "scatter"])), K=64)


@pytest.mark.parametrize("seed", range(24))
def test_oracle_matches_bruteforce(orc, seed):
    case = _random_case(seed)
    out, lse, _ = orc.attention(case)
    bout, blse = bruteforce.attention(case)
    assert np.all(np.isfinite(out)), "oracle read a poisoned row"
    assert _close(out, bout) and _close(lse, blse)


PAGE_EDGE = [  # (seq_lens, n_q, R, W) -- page edges, window edges, verify, multi-request
    ([255], 1, 0, 128), ([256], 1, 0, 128), ([257], 1, 0, 128), ([128], 1, 0, 128),
    ([260], 4, 0, 128), ([256], 16, 0, 128), ([33, 97], 1, 0, 128), ([300], 1, 0, 128),
    ([68], 1, 4, 128), ([80], 16, 4, 128), ([67, 99], 3, 4, 128),
    ([129], 1, 128, 128), ([144], 16, 128, 128), ([131, 163], 3, 128, 128),
]


@pytest.mark.parametrize("sl,nq,R,W", PAGE_EDGE)
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_oracle_matches_bruteforce_edges(orc, sl, nq, R, W, kv):
    case = make_case(seq_lens=sl, n_q=nq, H=3, R=R, W=W, kv=kv, seed=hash((tuple(sl), nq, R)) % 1000,
                     keep_logical=True, K=64)
    out, lse, _ = orc.attention(case)
    bout, blse = bruteforce.attention(case)
    assert _close(out, bout) and _close(lse, blse)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_single_key_closed_form(orc):
    case = make_case(seq_lens=[1], n_q=1, H=4, R=0, seed=5, keep_logical=True)
    out, lse, lse_ns = orc.attention(case)
    k = bruteforce.decode_rows(case.logical[0]["tok"])[0]
    q = bruteforce.bf16_bits_to_f64(case.q[0])
    s = case.scale * (q @ k)
    sig = case.sink.astype(np.float64)
    den = np.exp(s) + np.exp(sig)
    assert _close(out[0], (np.exp(s) / den)[:, None] * k[None, :])
    assert _close(lse[0], np.log(den))
    assert _close(lse_ns[0], s)


@pytest.mark.parametrize("R,sl,nq", [(0, [90, 500], [1, 2]), (128, [700], [3]), (4, [333, 65], [2, 1])])
def test_identical_keys_closed_form(orc, R, sl, nq):
    """N identical value rows v: out = v * N e^s / (N e^s + e^sink)."""
    case = make_case(seq_lens=sl, n_q=nq, H=3, R=R, seed=11, K=64, n_sel=17)
    v_bits = case.q[0, 0].copy()
    case.swa_pool[:] = v_bits[None, :]
    if case.extra_pool is not None:
        case.extra_pool[:] = v_bits[None, :]
    out, lse, _ = orc.attention(case)
    v = bruteforce.bf16_bits_to_f64(v_bits)
    qs = bruteforce.bf16_bits_to_f64(case.q.reshape(-1, 512)).reshape(case.T, case.H, 512)
    for t in range(case.T):
        r = int(np.searchsorted(case.qo_indptr, t, side="right") - 1)
        p = int(case.seq_lens[r]) - int(case.qo_indptr[r + 1] - case.qo_indptr[r]) + t - int(case.qo_indptr[r])
        n = min(case.W, p + 1)
        if R == 128:
            n += (p + 1) // 128
        elif R == 4:
            n += int(np.sum(case.c4_indices[t] >= 0))
        s = case.scale * (qs[t] @ v)
        sig = case.sink.astype(np.float64)
        mass = n * np.exp(s) / (n * np.exp(s) + np.exp(sig))
        assert _close(out[t], mass[:, None] * v[None, :])
        assert _close(lse[t], np.log(n * np.exp(s) + np.exp(sig)))


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def _permute_pages(case, seed):
    rng = np.random.default_rng(seed)

    def perm_pool(pool, table, fp8):
        n_pages = pool.shape[0] if fp8 else pool.shape[0] // 256
        pi = rng.permutation(n_pages)
        pages = pool if fp8 else pool.reshape(n_pages, 256, 512)
        new = np.empty_like(pages)
        new[pi] = pages
        return (new if fp8 else new.reshape(-1, 512)), pi[table].astype(np.int32)

    fp8 = case.kv == "fp8"
    swa, swa_t = perm_pool(case.swa_pool, case.swa_page_table, fp8)
    ext, ext_t = case.extra_pool, case.extra_page_table
    if ext is not None:
        ext, ext_t = perm_pool(ext, ext_t, fp8)
    return dataclasses.replace(case, swa_pool=swa, swa_page_table=swa_t, extra_pool=ext, extra_page_table=ext_t)


@pytest.mark.parametrize("R,kv", [(0, "bf16"), (4, "fp8"), (128, "bf16")])
def test_page_permutation_bit_exact(orc, R, kv):
    case = make_case(seq_lens=[300, 520], n_q=[2, 3], H=2, R=R, kv=kv, seed=21, K=64)
    a = orc.attention(case)
    b = orc.attention(_permute_pages(case, 3))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _permute_requests(case, sigma):
    sigma = np.asarray(sigma)
    n_q = np.diff(case.qo_indptr)
    blocks = [np.arange(case.qo_indptr[r], case.qo_indptr[r + 1]) for r in sigma]
    rows = np.concatenate(blocks)
    qo = np.zeros(case.B + 1, np.int32)
    qo[1:] = np.cumsum(n_q[sigma])
    return dataclasses.replace(
        case,
        seq_lens=case.seq_lens[sigma],
        qo_indptr=qo,
        q=case.q[rows],
        swa_page_table=case.swa_page_table[sigma],
        extra_page_table=None if case.extra_page_table is None else case.extra_page_table[sigma],
        c4_indices=None if case.c4_indices is None else case.c4_indices[rows],
    ), rows


def test_request_permutation_permutes_rows(orc):
    case = make_case(seq_lens=[300, 40, 520], n_q=[2, 1, 3], H=2, R=4, seed=8, K=64)
    perm_case, rows = _permute_requests(case, [2, 0, 1])
    a = orc.attention(case)
    b = orc.attention(perm_case)
    for x, y in zip(a, b):
        assert np.array_equal(x[rows], y)


def test_sink_neg_inf_is_plain_softmax(orc):
    base = make_case(seq_lens=[300], n_q=2, H=3, R=128, seed=4, sink=False)
    out0, lse0, ns0 = orc.attention(base)
    assert np.array_equal(lse0, ns0)
    tiny = dataclasses.replace(base, sink=np.full(3, -1e30, np.float32))
    out1, lse1, _ = orc.attention(tiny)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)
    ninf = dataclasses.replace(base, sink=np.full(3, -np.inf, np.float32))
    out2, lse2, _ = orc.attention(ninf)
    assert np.array_equal(out0, out2) and np.array_equal(lse0, lse2)


def test_sink_zero_changes_result(orc):
    base = make_case(seq_lens=[50], n_q=1, H=2, R=0, seed=4, sink=True, sink_value=0.0)
    out, lse, ns = orc.attention(base)
    assert np.all(lse > ns)
    assert np.allclose(lse, np.logaddexp(ns, 0.0), rtol=0, atol=1e-13)


def test_c4_without_indices_equals_swa_only(orc):
    c4 = make_case(seq_lens=[300, 90], n_q=[2, 1], H=2, R=4, seed=9, K=64)
    c4.c4_indices[:] = -1
    swa = dataclasses.replace(c4, R=0, c4_indices=None, extra_pool=None, extra_page_table=None)
    for x, y in zip(orc.attention(c4), orc.attention(swa)):
        assert np.array_equal(x, y)


def test_c128_before_first_block_equals_swa_only(orc):
    c = make_case(seq_lens=[127, 100], n_q=[3, 1], H=2, R=128, seed=9)
    swa = dataclasses.replace(c, R=0, extra_pool=None, extra_page_table=None)
    for x, y in zip(orc.attention(c), orc.attention(swa)):
        assert np.array_equal(x, y)


def test_swa_within_window_equals_full_causal(orc):
    case = make_case(seq_lens=[128, 77], n_q=[5, 2], H=2, R=0, seed=12, keep_logical=True)
    out, lse, _ = orc.attention(case)
    fout, flse = bruteforce.attention(case, window=10 ** 9)
    assert _close(out, fout) and _close(lse, flse)


def test_fp8_exact_values_equal_bf16(orc):
    """E4M3 code x power-of-two scale is exact in bf16, so both formats must agree bit for bit."""
    c8 = make_case(seq_lens=[300, 700], n_q=[1, 2], H=2, R=4, kv="fp8", seed=13, K=64, n_sel=40, keep_logical=True)
    from synth.workloads import FP8_SCALE_OFFSET

    c8.swa_pool[:, FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 1024] = np.full(256, 0.125, np.float32).view(np.uint8)
    c8.extra_pool[:, FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 1024] = np.full(256, 0.125, np.float32).view(np.uint8)

    def to_bf16_pool(pool):
        n_pages = pool.shape[0]
        rec = pool[:, :FP8_SCALE_OFFSET].reshape(n_pages * 256, 576)
        nope = torch.from_numpy(np.ascontiguousarray(rec[:, :448])).view(torch.float8_e4m3fn).to(torch.float32) * 0.125
        rope = torch.from_numpy(np.ascontiguousarray(rec[:, 448:]).view(np.int16)).view(torch.bfloat16)
        rows = torch.cat([nope.to(torch.bfloat16), rope], dim=1)
        return rows.view(torch.int16).numpy().view(np.uint16).copy()

    cb = dataclasses.replace(c8, kv="bf16", swa_pool=to_bf16_pool(c8.swa_pool), extra_pool=to_bf16_pool(c8.extra_pool))
    for x, y in zip(orc.attention(c8), orc.attention(cb)):
        assert np.array_equal(x, y)


def test_caller_contract_errors(orc):
    case = make_case(seq_lens=[300], n_q=1, H=1, R=4, seed=1, K=8, n_sel=4)
    bad = dataclasses.replace(case, c4_indices=case.c4_indices.copy())
    bad.c4_indices[0, 0] = 10 ** 6
    with pytest.raises(oracle_mod.OracleError, match="not visible"):
        orc.attention(bad)
    bad2 = dataclasses.replace(case, swa_page_table=np.full_like(case.swa_page_table, -1))
    with pytest.raises(oracle_mod.OracleError, match="outside pool"):
        orc.attention(bad2)


# --------------------------------------------------------------------------
# worked examples printed by the DSV4 walk-through page
# --------------------------------------------------------------------------
def _positions_from_gather(orc, case):
    pos = []
    for t in range(case.T):
        swa, _ = orc.gather(case, t)
        r = int(np.searchsorted(case.qo_indptr, t, side="right") - 1)
        base = int(case.swa_page_table[r, 0]) * 256
        pos.append([int(s) - base for s in swa])
    return pos


def test_walkthrough_worked_examples(orc):
    g = json.load(open(os.path.join(GOLDEN, "walkthrough_positions.json")))
    dec = g["printed"]["decode"]
    case = make_case(seq_lens=dec["seq_lens"], n_q=1, H=1, R=0, W=128, seed=2)
    assert case.qo_indptr.tolist() == dec["qo_indptr"]
    pos = _positions_from_gather(orc, case)
    assert [p[-1] for p in pos] == dec["positions"]
    assert all(p == list(range(p[-1] + 1)) for p in pos)

    pre = g["printed"]["prefill"]
    case = make_case(seq_lens=pre["total_lens"], n_q=pre["new_lens"], H=1, R=0, W=128, seed=2)
    assert case.qo_indptr.tolist() == pre["qo_indptr"]
    pos = _positions_from_gather(orc, case)
    assert [p[-1] for p in pos] == g["derived_reading"]["prefill_positions"]


# --------------------------------------------------------------------------
# mutants: a plausible mistake anywhere must fail a pin
# --------------------------------------------------------------------------
MUTANTS = {
    1: "window one token too wide", 2: "row positions shifted", 3: "sink multiplied by scale",
    4: "sink missing from the denominator", 5: "rotary dims missing from scores",
    6: "fp8 scale not applied", 7: "C128 last complete block hidden", 8: "page/offset swapped",
    9: "verify rows share the first row's C4 list", 10: "lse without the sink",
    11: "value without rotary dims", 12: "score scale not applied",
}

BATTERY = [
    dict(seq_lens=[5, 300], n_q=[1, 3], H=2, R=0, W=3),
    dict(seq_lens=[130, 385, 640], n_q=[1, 4, 2], H=3, R=128, W=4),
    dict(seq_lens=[200, 513], n_q=[1, 4], H=2, R=4, W=128, kv="fp8", K=64, n_sel=40, pad_mode="scatter"),
    dict(seq_lens=[260], n_q=[2], H=2, R=0, W=128),
]


def _battery_passes(o):
    for i, kw in enumerate(BATTERY):
        case = make_case(seed=100 + i, keep_logical=True, **kw)
        try:
            out, lse, _ = o.attention(case)
        except oracle_mod.OracleError:
            return False
        bout, blse = bruteforce.attention(case)
        if not (_close(out, bout) and _close(lse, blse)):
            return False
    return True


def test_battery_passes_on_oracle(orc):
    assert _battery_passes(orc)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path_factory, mutant):
    d = str(tmp_path_factory.mktemp(f"m{mutant}"))
    path = oracle_mod.build(mutant=mutant, out_dir=d)
    o = oracle_mod.Oracle(path)
    assert o.lib.dsv4o_mutant() == mutant
    assert not _battery_passes(o), f"mutant {mutant} ({MUTANTS[mutant]}) survived the pins"
