"""Pins of the oracle's E4M3 and bf16 codecs (CPU only).

The E4M3 table is pinned to the format facts the pages print
(tests/golden/page_facts.json), to an exhaustive round trip, to brute-force
nearest search in exact rational arithmetic, and to torch's own
float8_e4m3fn / bfloat16 casts (an independent library implementation).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_decode_format_facts():
    t = e4m3.DECODE_TABLE
    assert t[0x7E] == GOLDEN["e4m3_max"]["value"] == 448.0
    assert np.nanmax(np.abs(t)) == 448.0
    assert t[0x08] == GOLDEN["e4m3_min_normal"]["value"]   # smallest normal 2^-6
    assert t[0x01] == 2.0 ** -9                            # smallest subnormal
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert np.isfinite(np.delete(t, [0x7F, 0xFF])).all()   # no infinities ("fn")
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                        # codes ascend
    np.testing.assert_array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE_TABLE
    nan = np.isnan(ref)
    np.testing.assert_array_equal(nan, np.isnan(ours))
    np.testing.assert_array_equal(ref[~nan], ours[~nan])


def test_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3.encode(e4m3.decode(codes)), codes)


@pytest.mark.parametrize("value,expected", [
    (2.0 ** -10, 0x00),          # tie 0 | 2^-9 -> even code 0x00
    (3 * 2.0 ** -10, 0x02),      # tie 2^-9 | 2^-8 -> even code 0x02 (= 2^-8)
    (7.5 * 2.0 ** -9, 0x08),     # tie at the subnormal/normal boundary -> 2^-6
    (432.0, 0x7E),               # tie 416 | 448 -> even code 0x7E (= 448)
    (-432.0, 0xFE),
    (-0.0, 0x80),                # sign of zero kept
    (-(2.0 ** -11), 0x80),       # negative value rounding to zero keeps its sign
    (448.0, 0x7E),
])
def test_encode_ties_and_signs(value, expected):
    assert int(e4m3.encode(np.array([value]))[0]) == expected


def _brute_nearest(v: float) -> int:
    """Exact nearest finite code by rational arithmetic; ties -> even code."""
    fv = Fraction(v)
    best = None
    for c in range(0x7F):
        d = abs(abs(fv) - Fraction(e4m3.DECODE_TABLE[c]))
        key = (d, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    code = best[1]
    return code | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_encode_brute_force_rational():
    rng = np.random.default_rng(0)
    mags = np.concatenate([
        rng.uniform(0, 448, 300), rng.uniform(0, 2.0 ** -5, 300),
        np.ldexp(rng.uniform(1, 2, 200), rng.integers(-12, 9, 200)),
    ]).astype(np.float32)
    signs = rng.choice([-1.0, 1.0], mags.size).astype(np.float32)
    vals = np.clip(mags * signs, -448, 448)
    got = e4m3.encode(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        assert g == _brute_nearest(v), v


def test_encode_all_bf16_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.to_f32(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    vals = vals[keep]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3.encode(vals), ref)


def test_encode_fp32_near_midpoints_vs_torch():
    pos = e4m3.DECODE_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = [mids]
    up, dn = mids.copy(), mids.copy()
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        vals += [up, dn]
    vals = np.concatenate(vals)
    vals = vals[np.abs(vals) <= 448]
    vals = np.concatenate([vals, -vals])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3.encode(vals), ref)


def test_encode_random_fp32_vs_torch():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        np.ldexp(rng.uniform(-2, 2, 200_000), rng.integers(-20, 8, 200_000)),
    ]).astype(np.float32)
    vals = np.clip(vals, -448, 448)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3.encode(vals), ref)


def test_encode_relative_error_bound():
    # 3 mantissa bits: at most 2^-4 relative error in the normal range
    bound = GOLDEN["relative_error_bound"]["value"]
    rng = np.random.default_rng(2)
    v = np.ldexp(rng.uniform(1, 2, 100_000), rng.integers(-6, 8, 100_000))
    v = np.clip(v, 2.0 ** -6, 448)
    err = np.abs(e4m3.decode(e4m3.encode(v)) - v) / v
    assert err.max() <= bound
    assert err.max() > 0.9 * bound       # the bound is attained, not loose


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([449.0]))
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan]))


# --------------------------------------------------------------------------- bf16

def test_bf16_round_vs_torch_random():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(100_000),
        np.ldexp(rng.uniform(1, 2, 50_000), rng.integers(-140, 127, 50_000)),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16.round_from_f64(v.astype(np.float64)), ref)


def test_bf16_round_ties_and_edges():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: 0x3F80,          # tie -> even (1.0)
        one + 3 * ulp / 2: 0x3F82,      # tie -> even (1 + 2 ulp)
        -(one + ulp / 2): 0xBF80,
        2.0 ** -133: 0x0001,            # smallest subnormal
        2.0 ** -134: 0x0000,            # tie with 0 -> even (0)
        3 * 2.0 ** -134: 0x0002,        # tie 1|2 subnormal steps -> even
        bf16.BF16_MAX: 0x7F7F,
        2.0 ** 128: 0x7F80,             # overflow -> inf
        (2.0 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,   # tie max|inf rounds to even (inf)
        -0.0: 0x8000,
    }
    for v, bits in cases.items():
        assert int(bf16.round_from_f64(np.array([v]))[0]) == bits, v


def test_bf16_round_single_rounding_from_f64():
    # a value just above a bf16 midpoint by less than an fp32 ulp: a double
    # rounding through fp32 would land on the tie and go to even (down)
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert int(bf16.round_from_f64(np.array([v]))[0]) == 0x3F81
