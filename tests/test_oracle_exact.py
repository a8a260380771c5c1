"""Exact pins of the two quotient roundings of the quantize formula (CPU only).

The pages define the activation scale as s = amax / 448 and the code as
q = clamp(round(x / s), -448, 448) with round-to-nearest-even ([SGL19]
"从浮点到 FP8 的基本公式"; [GLM17] "第 1 站:RMSNorm 的两个出口").  With an
fp32 scale both quotients are single IEEE fp32 roundings (the oracle's
readings (i) and (ii)).  Those roundings are pinned here against the exact
rationals (``tests/exact_arith.py``: integer division with remainder,
brute-force nearest E4M3), over every input the quantizers can see:

* the scale: every positive finite bf16 amax, the fp32 floor 1e-10 and
  values below it;
* the code: every (amax, x) pair of bf16 values with |x| <= amax over the
  top 24 binades below amax, for every bf16 significand of amax (codes and
  scales are invariant under power-of-two scaling of a group, so one binade
  of amax stands for all), both signs, plus groups below the floor;
* the static quantizer: random fp32 scales, including saturating ones.

A reciprocal multiply in place of either division (x * RN32(1/s),
amax * RN32(1/448)) changes many of these results, so it fails here
(``test_oracle_mutations.py`` plants both).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant
from tests.exact_arith import e4m3_nearest, quantize_exact, rn32_quotient

FLOOR = np.float32(1e-10)


def _rn32_fraction(q: Fraction) -> float:
    """Independent slow RN32 of a rational (normal range), for the helper's own pin."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = q / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * float(lo * ulp)


def _all_positive_bf16() -> np.ndarray:
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def _bf16_binade(lo_exp: int, hi_exp: int) -> np.ndarray:
    """All bf16 values in [2^lo_exp, 2^hi_exp)."""
    m = np.arange(128, dtype=np.float64)
    e = np.arange(lo_exp, hi_exp, dtype=np.float64)
    return np.ldexp(1.0 + m[None, :] / 128.0, e[:, None].astype(np.int64)).reshape(-1).astype(np.float32)


# ----------------------------------------------------- the exact helper itself

def test_exact_quotient_agrees_with_fractions():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal(3000).astype(np.float32) * 100).to(torch.bfloat16).float().numpy()
    s = np.abs(rng.standard_normal(3000).astype(np.float32)) + np.float32(1e-3)
    # values chosen to give exact ties in the fp32 rounding
    x = np.concatenate([x, np.float32([1 + 2 ** -23, 3.0, 1.0, -5.0])])
    s = np.concatenate([s, np.float32([2.0, 3.0, 1.5, 7.0])])
    got = rn32_quotient(x, s)
    ref = np.array([_rn32_fraction(Fraction(float(a)) / Fraction(float(b))) for a, b in zip(x, s)])
    np.testing.assert_array_equal(got, ref)
    # and with IEEE hardware division (a third, unrelated route) on normal results
    np.testing.assert_array_equal(got, (x / s).astype(np.float32).astype(np.float64))


def test_exact_quotient_subnormal_and_overflow():
    x = np.float32([2.0 ** -140, 1e-45, 3e38, -3e38])
    s = np.float32([2.0 ** 10, 3.0, 2.0 ** -10, 2.0 ** -10])
    np.testing.assert_array_equal(rn32_quotient(x, s), (x / s).astype(np.float32).astype(np.float64))


def test_exact_e4m3_nearest_agrees_with_torch_cast():
    rng = np.random.default_rng(1)
    t = rng.uniform(-448, 448, 200_000).astype(np.float32)
    v = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)          # exact ties
    t = np.concatenate([t, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -11])])
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_nearest(t.astype(np.float64)), ref)


# ------------------------------------------------------------- the group scale

def check_group_scale(fn):
    """fn(amax) must equal RN32(max(amax, fp32(1e-10)) / 448) for every input."""
    a = np.concatenate([_all_positive_bf16(), np.float32([FLOOR, 0.0, 1e-12, 9.99e-11])])
    exact = rn32_quotient(np.maximum(a, FLOOR), np.float32(448.0))
    got = np.asarray(fn(a), np.float32).astype(np.float64)
    bad = np.nonzero(got != exact)[0]
    assert bad.size == 0, f"{bad.size} scales differ, e.g. amax={a[bad[0]]!r}"


def test_group_scale_exact_for_every_bf16_amax():
    check_group_scale(quant.group_scale)


# -------------------------------------------------------------- the code bytes

def _pairs():
    """(x, s) over the quantizer's domain: every amax significand in [1, 2),
    every bf16 |x| <= amax down to 2^-24 amax, both signs."""
    amax = _bf16_binade(0, 1)                                  # 128 values
    xs = _bf16_binade(-24, 1)
    X, A = np.meshgrid(xs, amax, indexing="xy")
    keep = X <= A
    x = X[keep]
    a = A[keep]
    x = np.concatenate([x, -x])
    a = np.concatenate([a, a])
    return x.astype(np.float32), a.astype(np.float32)


def check_quantize_with_scale(fn):
    x, a = _pairs()
    s = rn32_quotient(a, np.float32(448.0)).astype(np.float32)  # the scale the code sees
    ref = quantize_exact(x, s)
    got = np.asarray(fn(x, s), np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} of {x.size} codes differ, e.g. x={x[bad[0]]!r} s={s[bad[0]]!r}"


def test_quantize_with_scale_exact_over_the_group_domain():
    check_quantize_with_scale(quant.quantize_with_scale)


def test_quant_group_end_to_end_exact():
    # groups built from the domain above: each row one group of 128, its
    # first element the amax, the rest drawn from values at most amax
    rng = np.random.default_rng(2)
    amax = _bf16_binade(-3, 3)
    xs = _bf16_binade(-30, 3)
    rows = []
    for a in amax:
        pool = xs[xs <= a]
        v = rng.choice(pool, 127) * rng.choice(np.float32([-1, 1]), 127)
        rows.append(np.concatenate([[a], v]))
    x = np.array(rows, np.float32)
    x[::3, 0] = -x[::3, 0]                                   # amax from a negative value
    # groups whose amax is below the floor, and an all-zero group
    tiny = np.full((3, 128), 0.0, np.float32)
    tiny[0] = np.ldexp(np.float32(1.5), -36) * rng.choice(np.float32([-1, 1, 0.5]), 128)
    tiny[1, :5] = np.float32([9e-11, -5e-11, 1e-12, 0, -0.0])
    x = np.concatenate([x, tiny])
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    q, s = quant.quant_group(x)
    a = np.maximum(np.abs(x).max(axis=1), FLOOR)
    s_ref = rn32_quotient(a, np.float32(448.0))
    np.testing.assert_array_equal(s[:, 0].astype(np.float64), s_ref)
    np.testing.assert_array_equal(q, quantize_exact(x, s_ref.astype(np.float32)[:, None]))


def test_static_quant_exact_with_saturation():
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((64, 512)).astype(np.float32) * 30).to(torch.bfloat16).float().numpy()
    for s in (np.float32(0.0371), np.float32(1.0), np.float32(0.013), np.float32(3.3e-3)):
        q = quant.quant_static(x, s)
        np.testing.assert_array_equal(q, quantize_exact(x, s))
    assert (quant.quant_static(x, np.float32(3.3e-3)) & 0x7F == 0x7E).any()     # saturated codes present


def test_division_forms_differ_often_on_the_domain():
    # the readings matter: a reciprocal multiply gives other codes and scales
    x, a = _pairs()
    s = rn32_quotient(a, np.float32(448.0)).astype(np.float32)
    recip = (x * (np.float32(1) / s).astype(np.float32)).astype(np.float32)
    alt = e4m3_nearest(np.clip(recip.astype(np.float64), -448, 448))
    diff = np.count_nonzero(alt != quantize_exact(x, s))
    assert diff > 100, diff
    b = _all_positive_bf16()
    alt_s = (np.maximum(b, FLOOR) * (np.float32(1) / np.float32(448))).astype(np.float32)
    assert np.count_nonzero(alt_s.astype(np.float64) != rn32_quotient(np.maximum(b, FLOOR), np.float32(448))) > 1000


@pytest.mark.parametrize("seed", [0])
def test_reciprocal_code_rate_on_normal_groups(seed):
    """Context for the readings: on N(0,1) bf16 groups of 128 the two forms
    of x/s give different codes for about one element in two thousand."""
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((4096, 1024)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    g = x.reshape(-1, 128)
    s = quant.group_scale(np.abs(g).max(axis=1))[:, None]
    q_div = quant.quantize_with_scale(g, s)
    q_rec = quant.e4m3.encode(np.clip((g * (np.float32(1) / s).astype(np.float32)).astype(np.float32), -448, 448))
    rate = np.count_nonzero(q_div != q_rec) / g.size
    assert 1e-4 < rate < 2e-3, rate
