"""Pins of the oracle's FP8 KV packer (CPU only).

The packer quantises K rows into the packed FP8 record (the cache write of the
DSV4 walk-through page, section 3; the 584-byte FP8 + bf16 record of the
SGLang DSV4 test-matrix page).  Pinned against things other than itself:

* torch's float32 -> float8_e4m3fn conversion (round to nearest even) for
  every in-range value tried: all finite codes, every midpoint between
  neighbours (ties), random magnitudes over the whole range;
* closed forms: saturation above 448, signed zeros, the round-trip error
  bound (at most half a step), a constant row (all codes +-448), a zero row
  (scale 1), the scale of a row with one large entry;
* the byte layout of a record: codes, rotary bf16 bits, the page's fp32
  scale, skipped slots and untouched bytes;
* the seeded generator's own packer (synth) on the same rows;
* mutants: deliberately wrong builds of the packer must fail the battery.
"""
import numpy as np
import pytest
import torch

import oracle as oracle_mod
from synth.workloads import FP8_PAGE_BYTES, FP8_ROW_BYTES, FP8_SCALE_OFFSET, _to_bf16_bits, _to_e4m3_codes


@pytest.fixture(scope="module")
def orc():
    oracle_mod.build()
    return oracle_mod.Oracle()


def _torch_codes(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _finite_values() -> np.ndarray:
    codes = np.array([c for c in range(128) if c != 0x7F], np.uint8)
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()


def _encode(orc, xs) -> np.ndarray:
    return np.array([orc.e4m3_from_float(float(x)) for x in np.asarray(xs, np.float32)], np.uint8)


def test_encoder_matches_torch_on_codes_midpoints_and_random(orc):
    v = _finite_values()                                     # 0 .. 448, ascending
    mids = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (v[:-1].astype(np.float64) + v[1:]) / 2)  # exact in float
    rng = np.random.default_rng(7)
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 4000)).astype(np.float32)
    xs = np.concatenate([v, mids, rand, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    assert np.array_equal(_encode(orc, xs), _torch_codes(xs))


def test_encoder_saturates_and_keeps_the_sign(orc):
    for x in (448.0, 455.0, 464.0, 479.9, 480.0, 1e4, 3e38):
        assert orc.e4m3_from_float(x) == 0x7E
        assert orc.e4m3_from_float(-x) == 0xFE
    assert orc.e4m3_from_float(0.0) == 0x00
    assert orc.e4m3_from_float(-0.0) == 0x80
    assert orc.e4m3_from_float(-2.0 ** -11) == 0x80   # rounds to zero, keeps the sign
    assert orc.e4m3_from_float(2.0 ** -10) == 0x00    # tie between 0 and 2^-9: the even code
    assert orc.e4m3_from_float(3 * 2.0 ** -10) == 0x02  # tie between 2^-9 and 2^-8: the even code


def test_encoder_round_trip_within_half_a_step(orc):
    rng = np.random.default_rng(8)
    xs = rng.uniform(-448, 448, 3000).astype(np.float32)
    v = np.concatenate([-_finite_values()[::-1], _finite_values()]).astype(np.float64)
    for x, c in zip(xs, _encode(orc, xs)):
        dec = orc.e4m3_to_double(int(c))
        i = np.searchsorted(v, float(x))
        lo, hi = v[max(i - 1, 0)], v[min(i, len(v) - 1)]
        assert abs(dec - float(x)) <= (hi - lo) / 2 + 0.0
        assert dec in (lo, hi)


def _rows(rng, n, big=None):
    k = rng.standard_normal((n, 512)).astype(np.float32)
    if big is not None:
        k[:, big] *= 300.0
    return _to_bf16_bits(k)


def _pack(orc, k_bits, slots, pages=3):
    pool = np.full((pages, FP8_PAGE_BYTES), 0xA5, np.uint8)
    orc.pack_fp8(k_bits, np.asarray(slots, np.int32), pool)
    return pool


def _record(pool, slot):
    page, rec = divmod(int(slot), 256)
    codes = pool[page, rec * FP8_ROW_BYTES: rec * FP8_ROW_BYTES + 448]
    rope = pool[page, rec * FP8_ROW_BYTES + 448: (rec + 1) * FP8_ROW_BYTES].view(np.uint16)
    scale = pool[page, FP8_SCALE_OFFSET + 4 * rec: FP8_SCALE_OFFSET + 4 * rec + 4].view(np.float32)[0]
    return codes, rope, scale


def test_record_layout_and_skipped_slots(orc):
    rng = np.random.default_rng(9)
    k = _rows(rng, 4)
    slots = [3, -1, 256 + 17, 2 * 256 + 255]
    pool = _pack(orc, k, slots)
    touched = np.zeros_like(pool, dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        codes, rope, scale = _record(pool, s)
        nope = k[i, :448].astype(np.uint32) << 16
        nope = nope.view(np.float32)
        assert scale == np.float32(np.abs(nope).max()) / np.float32(448.0)
        assert np.array_equal(codes, _torch_codes(nope / scale))
        assert np.array_equal(rope, k[i, 448:])
        page, rec = divmod(s, 256)
        touched[page, rec * FP8_ROW_BYTES:(rec + 1) * FP8_ROW_BYTES] = True
        touched[page, FP8_SCALE_OFFSET + 4 * rec:FP8_SCALE_OFFSET + 4 * rec + 4] = True
    assert np.all(pool[~touched] == 0xA5)


def test_closed_form_rows(orc):
    k = np.zeros((4, 512), np.float32)
    k[0, :448] = 0.75              # constant row: every code is the top code
    k[1, :448] = -3.0
    k[2, 448:] = 1.5               # zero non-rotary part: scale 1, zero codes
    k[3, :448] = 2.0 ** -20        # tiny constant row: still the top code
    k[3, 5] = -(2.0 ** -18)
    bits = _to_bf16_bits(k)
    pool = _pack(orc, bits, [0, 1, 2, 3], pages=1)
    c, _, s = _record(pool, 0)
    assert s == np.float32(0.75) / np.float32(448) and np.all(c == 0x7E)
    c, _, s = _record(pool, 1)
    assert s == np.float32(3.0) / np.float32(448) and np.all(c == 0xFE)
    c, r, s = _record(pool, 2)
    assert s == 1.0 and np.all(c == 0) and np.array_equal(r, bits[2, 448:])
    c, _, s = _record(pool, 3)
    assert s == np.float32(2.0 ** -18) / np.float32(448) and c[5] == 0xFE
    assert np.all(c[np.arange(448) != 5] == _torch_codes(np.float32([2.0 ** -20]) / s)[0])


def test_matches_the_generators_packer(orc):
    """synth quantises float32 rows with torch (RNE after a +-448 clamp); on
    rows that are bf16 values the two packers must write the same bytes."""
    rng = np.random.default_rng(10)
    bits = _rows(rng, 64, big=np.arange(0, 448, 37))
    nope = (bits[:, :448].astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(nope).max(axis=1)
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    want = _to_e4m3_codes(nope / scales[:, None])
    pool = _pack(orc, bits, np.arange(64))
    for i in range(64):
        codes, rope, scale = _record(pool, i)
        assert scale == scales[i]
        assert np.array_equal(codes, want[i])
        assert np.array_equal(rope, bits[i, 448:])


# --------------------------------------------------------------------------
# mutants: a plausible packer mistake must fail the battery
# --------------------------------------------------------------------------
PACK_MUTANTS = {13: "ties rounded away from zero", 14: "scale divisor 447", 15: "rotary dims swapped in pairs"}


def _pack_battery_passes(o):
    v = _finite_values()
    mids = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)
    if not np.array_equal(_encode(o, mids), _torch_codes(mids)):
        return False
    rng = np.random.default_rng(11)
    bits = _rows(rng, 8)
    nope = (bits[:, :448].astype(np.uint32) << 16).view(np.float32)
    scales = (np.abs(nope).max(axis=1) / np.float32(448.0)).astype(np.float32)
    pool = _pack(o, bits, np.arange(8), pages=1)
    for i in range(8):
        codes, rope, scale = _record(pool, i)
        if scale != scales[i] or not np.array_equal(rope, bits[i, 448:]):
            return False
        if not np.array_equal(codes, _torch_codes(nope[i] / scales[i])):
            return False
    return True


def test_pack_battery_passes_on_oracle(orc):
    assert _pack_battery_passes(orc)


@pytest.mark.parametrize("mutant", sorted(PACK_MUTANTS))
def test_pack_mutant_is_caught(tmp_path_factory, mutant):
    d = str(tmp_path_factory.mktemp(f"pm{mutant}"))
    o = oracle_mod.Oracle(oracle_mod.build(mutant=mutant, out_dir=d))
    assert o.lib.dsv4o_mutant() == mutant
    assert not _pack_battery_passes(o), f"mutant {mutant} ({PACK_MUTANTS[mutant]}) survived the pins"
