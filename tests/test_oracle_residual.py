"""Pins of the oracle's residual add -> RMSNorm -> quantization front end (CPU only).

The residual add is pinned against exact rational arithmetic; the fused
pipeline against a closed form (rows whose sum is constant), invariants that
follow from the reading that the norm reads the stored bf16 stream (symmetry
in the two addends, re-adding zero to the stored stream), a reduction to the
already pinned RMSNorm quantizer (zero sublayer output) and, for the static
exit, exact power-of-two scales.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, quant


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _bf16_round_exact(v: Fraction) -> float:
    """Nearest bf16 of a rational, ties to even, from the definition (8
    significant bits, exponent floor -126, overflow at 2^128 - 2^119)."""
    if v == 0:
        return 0.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 7)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * quantum
    if r >= Fraction(2) ** 128:
        return math.copysign(math.inf, v)
    return math.copysign(float(r), v)


def _pairs(n, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n)))
    gap = rng.integers(0, 40, n)
    h = _bf16(rng.standard_normal(n) * np.abs(x) * np.exp2(-gap.astype(np.float64)))
    # exact ties (half an ulp of x) and values just past them
    x[:8] = [1.0, 1.0 + 2.0 ** -7, -3.0, 1.5, 2.0 ** -126, -(2.0 ** -130), 3.0e38, -1.0]
    h[:8] = [2.0 ** -8, 2.0 ** -8, -(2.0 ** -7) * 3 / 2, 2.0 ** -8 * (1 + 2.0 ** -7),
             2.0 ** -133, 2.0 ** -133, 3.0e38, 1.0]
    return x.astype(np.float32), h.astype(np.float32)


def test_residual_add_is_correctly_rounded():
    x, h = _pairs(4000, 0)
    z = bf16.to_f64(quant.residual_add(x, h))
    for i in range(len(x)):
        exact = Fraction(float(x[i])) + Fraction(float(h[i]))
        assert z[i] == _bf16_round_exact(exact), (i, x[i], h[i], z[i])
    # the tie cases: 1 + 2^-8 -> 1 (even), (1 + 2^-7) + 2^-8 -> 1 + 2^-6, overflow -> inf, x - x -> +0
    assert z[0] == 1.0 and z[1] == 1.0 + 2.0 ** -6 and math.isinf(z[6])
    assert quant.residual_add(np.float32([-1.0]), np.float32([1.0]))[0] == 0x0000


def _norm_problem(M, K, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((M, K)))
    h = _bf16(rng.standard_normal((M, K)) * 0.25)
    g = _bf16(rng.uniform(0.5, 1.5, K))
    return x, h, g


def test_constant_sum_rows_closed_form():
    # x = k/16, h = c - x with c = 1.5: both bf16 and the sum is exactly c
    K, eps, c = 384, 1e-6, 1.5
    k = np.arange(K) % 129 - 64
    x = (k / 16.0).astype(np.float32)[None, :]
    h = (c - k / 16.0).astype(np.float32)[None, :]
    assert np.all(_bf16(x) == x) and np.all(_bf16(h) == h)
    g = _bf16(np.linspace(0.5, 1.5, K))
    out = quant.add_rmsnorm_quant(x, h, g, eps)
    assert np.all(bf16.to_f64(out["z"]) == c)
    r = np.float32(1.0 / math.sqrt(c * c + float(np.float32(eps))))
    assert out["r"][0] == r
    y = bf16.to_f64(out["y"])[0]
    assert np.all(np.abs(y - g) <= np.abs(g) * 2.0 ** -8)


def test_symmetric_in_stream_and_sublayer_output():
    x, h, g = _norm_problem(12, 640, 1)
    a = quant.add_rmsnorm_quant(x, h, g, 1e-6)
    b = quant.add_rmsnorm_quant(h, x, g, 1e-6)
    for key in ("z", "q", "s", "y"):
        np.testing.assert_array_equal(a[key], b[key])


def test_norm_reads_the_stored_stream():
    # adding a zero sublayer output to the stored stream changes nothing
    x, h, g = _norm_problem(16, 1000, 2)
    a = quant.add_rmsnorm_quant(x, h, g, 1e-6)
    b = quant.add_rmsnorm_quant(bf16.to_f32(a["z"]), np.zeros_like(x), g, 1e-6)
    for key in ("z", "q", "s", "y"):
        np.testing.assert_array_equal(a[key], b[key])


def test_zero_sublayer_output_is_rmsnorm_quant():
    x, _, g = _norm_problem(8, 768, 3)
    a = quant.add_rmsnorm_quant(x, np.zeros_like(x), g, 1e-6)
    b = quant.rmsnorm_quant(x, g, 1e-6)
    np.testing.assert_array_equal(a["z"], bf16.round_from_f64(x.astype(np.float64)))
    for key in ("q", "s", "y"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("k", [0, 4, 8])
def test_static_exit_power_of_two_scale(k):
    x, h, g = _norm_problem(6, 512, 4)
    s = np.float32(2.0 ** -k)
    out = quant.add_rmsnorm_quant(x, h, g, 1e-6, static_scale=s)
    assert out["s"] is None
    y = bf16.to_f64(out["y"])
    t = y * 2.0 ** k                                # exact: y / s
    codes = e4m3.encode(np.clip(t, -448.0, 448.0))
    np.testing.assert_array_equal(out["q"], codes)
    big = np.abs(t) >= 448.0
    if k == 8:
        assert big.any()                            # |y| above 1.75 saturates at 2^-8
    assert np.all((out["q"][big] & 0x7F) == 0x7E)


def test_dynamic_exit_group_scales_bound_the_stream():
    x, h, g = _norm_problem(10, 1280, 5)
    out = quant.add_rmsnorm_quant(x, h, g, 1e-6)
    deq = e4m3.decode(out["q"]).reshape(10, 10, 128) * out["s"][:, :, None].astype(np.float64)
    y = bf16.to_f64(out["y"]).reshape(10, 10, 128)
    # the largest element of each group maps to 448 exactly
    assert np.all(np.max(np.abs(e4m3.decode(out["q"]).reshape(10, 10, 128)), axis=2) == 448.0)
    assert np.all(np.abs(deq - y) <= np.abs(y) * 2.0 ** -4 + out["s"][:, :, None] * 2.0 ** -9 * 1.01)
