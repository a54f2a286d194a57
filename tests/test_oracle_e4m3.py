"""Pins of the oracle's E4M3 decode/encode against things other than itself.

* The pages fix 448 as the largest E4M3 value and 3 stored mantissa bits
  (tests/golden/page_constants.json); the OCP bit layout fixes the rest
  (tests/golden/e4m3_points.json, worked out by hand).
* torch's own float8_e4m3fn type is an independent library implementation of the same
  format: its decode must agree on all 256 codes, and its (non-saturating) round-to-nearest-
  even conversion must agree with the oracle's encoder wherever no saturation happens.
* The oracle carries two encoders written independently (binary32 bit surgery, and a search
  of the decode table with an explicit tie rule); they must agree on every binary32 input
  in the range where codes are not trivially zero or saturated.
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_float8_on_all_codes(orc):
    ours = orc.e4m3_decode_table()
    ref = _torch_decode_all()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert np.array_equal(np.flatnonzero(nan_ours), [0x7F, 0xFF])
    assert np.array_equal(ours[~nan_ours], ref[~nan_ours])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ours]))


def test_decode_properties_fixed_by_pages(orc):
    pc = _golden("page_constants.json")
    t = orc.e4m3_decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "0x00..0x7E must be strictly increasing"
    assert pos[-1] == pc["e4m3_max"]["value"] == np.nanmax(t)
    assert np.count_nonzero(pos > 0) == 126
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    # 3 stored mantissa bits: in every binade the 8 normal values step by 2^(E-7)/8
    mb = pc["e4m3_stored_mantissa_bits"]["value"]
    for e in range(1, 16):
        vals = t[(e << mb):(e << mb) + (1 << mb)]
        vals = vals[~np.isnan(vals)]
        steps = np.diff(vals)
        assert np.all(steps == 2.0 ** (e - 7) / 8)
    # provisional scale 2.0 covers |x| <= 896 = 2.0 * 448
    assert pc["provisional_scale"]["value"] * pos[-1] == pc["provisional_scale"]["covers_abs"]


def test_decode_golden_points(orc):
    t = orc.e4m3_decode_table()
    for code, val in _golden("e4m3_points.json")["decode"]:
        v = float(val)
        got = t[int(code, 16)]
        assert got == v and np.signbit(got) == np.signbit(v), (code, got, v)


@pytest.mark.parametrize("enc", ["e4m3_encode", "e4m3_encode_search"])
def test_encode_golden_points(orc, enc):
    f = getattr(orc, enc)
    for val, code, why in _golden("e4m3_points.json")["encode"]:
        got = int(f(np.array([float(val)], dtype=np.float32))[0])
        assert got == int(code, 16), (val, hex(got), code, why)


@pytest.mark.parametrize("enc", ["e4m3_encode", "e4m3_encode_search"])
def test_encode_roundtrips_every_finite_code(orc, enc):
    t = orc.e4m3_decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = t[codes].astype(np.float32)
    got = getattr(orc, enc)(vals)
    assert np.array_equal(got, codes)


def test_encode_saturates_instead_of_nan(orc):
    big = np.array([448.0, 448.5, 463.99, 464.0, 465.0, 480.0, 896.0, 1e6, 3.0e38],
                   dtype=np.float32)
    assert np.all(orc.e4m3_encode(big) == 0x7E)
    assert np.all(orc.e4m3_encode(-big) == 0xFE)
    assert np.all(orc.e4m3_encode_search(big) == 0x7E)
    assert np.all(orc.e4m3_encode_search(-big) == 0xFE)


def _chunks(lo, hi, parts):
    edges = np.linspace(lo, hi + 1, parts + 1).astype(np.int64)
    return [(int(a), int(b) - 1) for a, b in zip(edges[:-1], edges[1:])]


@pytest.mark.slow
def test_two_encoders_agree_on_every_binary32_in_range(orc):
    """Every binary32 pattern with |v| <= 512, both signs: zero, the binary32 subnormals and
    every normal value up to 512 (about 2.3e9 inputs)."""
    lo = 0
    hi = int(np.float32(512.0).view(np.uint32))
    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(lambda ab: orc.e4m3_sweep_compare(*ab), _chunks(lo, hi, 64)))
    bad = sum(r[0] for r in res)
    firsts = [hex(r[1]) for r in res if r[0]]
    assert bad == 0, firsts[:4]


def test_encode_matches_torch_rne_below_saturation(orc):
    """torch's float8_e4m3fn conversion rounds to nearest even and turns overflow into NaN;
    below 464 (half-way above 448) it never overflows, so there it must equal the oracle.
    Every binary32 pattern with 2^-12 <= |v| < 464 is checked, one 2^22 chunk at a time."""
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(464.0).view(np.uint32)) - 1
    step = 1 << 22
    for a in range(lo, hi + 1, step):
        bits = np.arange(a, min(a + step, hi + 1), dtype=np.uint32)
        v = bits.view(np.float32)
        for vv in (v, -v):
            ref = torch.from_numpy(vv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            got = orc.e4m3_encode(vv)
            if not np.array_equal(ref, got):
                i = int(np.flatnonzero(ref != got)[0])
                pytest.fail(f"v={vv[i]!r} torch={ref[i]:#x} oracle={got[i]:#x}")


def test_encode_tiny_values_match_torch(orc):
    """Below 2^-12 every value rounds to a signed zero; includes binary32 subnormals."""
    rng = np.random.default_rng(11)
    hi = int(np.float32(2.0 ** -12).view(np.uint32))
    bits = np.concatenate([rng.integers(0, hi, size=200000, dtype=np.uint32),
                           np.arange(0, 4096, dtype=np.uint32)])
    v = bits.view(np.float32)
    for vv in (v, -v):
        ref = torch.from_numpy(vv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(orc.e4m3_encode(vv), ref)
        assert np.array_equal(orc.e4m3_encode_search(vv), ref)
    assert np.all(orc.e4m3_encode(v) == 0) and np.all(orc.e4m3_encode(-v) == 0x80)
