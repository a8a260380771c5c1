"""Pins of the oracle's quantizers (CPU only).

Each pin is independent of the code it checks: invariants implied by the
pages' formulas, the byte accounting the pages print, exact special cases,
exhaustive enumeration, and torch library routines.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, quant
from tests.exact_arith import rn32_quotient

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _bf16_data(shape, seed, scale=1.0, outlier_cols=()):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32) * scale
    for c in outlier_cols:
        x[:, c] *= 50
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


# ------------------------------------------------------------- group quantizer

def test_group_max_code_is_448_in_every_group():
    x = _bf16_data((64, 1024), 0, outlier_cols=(5, 700))
    q, s = quant.quant_group(x)
    dq = np.abs(e4m3.decode(q)).reshape(64, 8, 128).max(axis=2)
    assert np.all(dq == 448.0)


def test_group_error_bound():
    # |q*s - x| <= 2^-4 |x| where |x/s| >= 2^-6, else half the subnormal step
    x = _bf16_data((128, 1024), 1, outlier_cols=(3,))
    q, s = quant.quant_group(x)
    S = np.repeat(s.astype(np.float64), 128, axis=1)
    dq = e4m3.decode(q) * S
    err = np.abs(dq - x)
    ratio = np.abs(x) / S
    slack = 1 + 2.0 ** -20          # fp32 division before the E4M3 rounding
    normal = ratio >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * slack)
    assert np.all(err[~normal] <= 2.0 ** -10 * S[~normal] * slack)
    rel_rms = math.sqrt(np.mean((err[normal] / np.abs(x[normal])) ** 2))
    # context only: the pages estimate ~1.8%; uniform mantissas give more
    assert 0.005 < rel_rms < GOLDEN["relative_error_bound"]["value"]


def test_group_scale_equals_amax_over_448():
    x = _bf16_data((16, 512), 2)
    _, s = quant.quant_group(x)
    amax = np.abs(x).reshape(16, 4, 128).max(axis=2)
    # the correctly rounded fp32 quotient, from exact rational arithmetic
    np.testing.assert_array_equal(s.astype(np.float64), rn32_quotient(amax, np.float32(448.0)))


def test_group_identity_on_representable_inputs():
    # inputs already E4M3 with a +-448 in every group -> s == 1, codes returned
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, size=(8, 384)).astype(np.uint8)
    for g in range(3):
        codes[:, g * 128 + rng.integers(0, 128)] = rng.choice([0x7E, 0xFE])
    x = e4m3.decode(codes).astype(np.float32)
    q, s = quant.quant_group(x)
    assert np.all(s == 1.0)
    np.testing.assert_array_equal(q, codes)


def test_group_power_of_two_equivariance():
    x = _bf16_data((32, 512), 4)
    q0, s0 = quant.quant_group(x)
    for k in (-20, -3, 5, 30):
        q1, s1 = quant.quant_group(np.ldexp(x, k))
        np.testing.assert_array_equal(q1, q0)
        np.testing.assert_array_equal(s1, np.ldexp(s0, k))


def test_group_ragged_tail_is_its_own_group():
    x = _bf16_data((4, 520), 5)
    q, s = quant.quant_group(x)
    assert s.shape == (4, 5)
    qt, st = quant.quant_group(x[:, 512:])
    np.testing.assert_array_equal(q[:, 512:], qt)
    np.testing.assert_array_equal(s[:, 4:], st)


def test_group_zero_group_uses_floor():
    x = np.zeros((2, 256), np.float32)
    x[1, 200] = 3.0
    q, s = quant.quant_group(x)
    floor_scale = np.float32(rn32_quotient(np.float32(1e-10), np.float32(448.0)))
    assert s[0, 0] == floor_scale and s[0, 1] == floor_scale and s[1, 0] == floor_scale
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert q[1, 200] == 0x7E


def test_group_negative_zero_and_tiny_negatives_keep_sign():
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 448.0
    x[0, 1] = -0.0
    x[0, 2] = -1e-6
    q, _ = quant.quant_group(x)
    assert q[0, 1] == 0x80 and q[0, 2] == 0x80 and q[0, 3] == 0x00


def test_group_rows_independent():
    x = _bf16_data((10, 384), 6)
    q, s = quant.quant_group(x)
    for i in (0, 7):
        qi, si = quant.quant_group(x[i:i + 1])
        np.testing.assert_array_equal(q[i:i + 1], qi)
        np.testing.assert_array_equal(s[i:i + 1], si)


def test_row_6144_byte_accounting():
    f = GOLDEN["row_6144"]
    x = _bf16_data((1, f["K"]), 7)
    q, s = quant.quant_group(x)
    assert s.shape[1] == f["groups"]
    assert q.nbytes + s.nbytes == f["bytes_quantized"]
    assert x.shape[1] * 2 == f["bytes_bf16"]


def test_scale_overhead_accounting():
    f = GOLDEN["scale_overhead"]
    for group, key in ((128, "group128"), (64, "group64")):
        x = _bf16_data((1, 1024), 8)
        q, s = quant.quant_group(x, group)
        assert s.nbytes / q.nbytes == f[key]
    assert round(100 * f["group128"], 1) == 3.1


def test_dispatch_scale_bytes_accounting():
    f = GOLDEN["dispatch_scale_bytes"]
    x = _bf16_data((1, f["K"]), 9)
    _, s = quant.quant_group(x, 128)
    assert s.nbytes == f["fp32_bytes"]
    assert s.size * 1 == f["ue8m0_bytes"]
    assert abs((f["fp32_bytes"] - f["ue8m0_bytes"]) / f["K"] - 0.0234375) < 1e-12


def test_static_quant_matches_division_rule():
    x = _bf16_data((8, 256), 10)
    sx = np.float32(np.abs(x).max() / np.float32(448))
    q = quant.quant_static(x, sx)
    # same codes as the group quantizer when every group shares that scale
    q2 = e4m3.encode(np.clip((x / sx).astype(np.float32), -448, 448))
    np.testing.assert_array_equal(q, q2)
    assert np.abs(e4m3.decode(q)).max() == 448.0


def test_static_quant_saturates_out_of_range():
    x = np.array([[1000.0, -1000.0, 1.0]], np.float32)
    q = quant.quant_static(x, np.float32(1.0))
    assert q.tolist() == [[0x7E, 0xFE, 0x38]]


# --------------------------------------------------------------- weight blocks

def test_weight_grid_7168x2048():
    f = GOLDEN["weight_grid_7168x2048"]
    w = np.zeros((f["N"], f["K"]), np.float32)
    _, s = quant.quant_weight_block(w)
    assert list(s.shape) == f["grid"] and s.size == f["count"]


def test_moe_scale_count():
    f = GOLDEN["moe_scale_count"]
    H, I = f["hidden"], f["intermediate"]
    _, s13 = quant.quant_weight_block(np.zeros((2 * I, H), np.float32))
    _, s2 = quant.quant_weight_block(np.zeros((H, I), np.float32))
    assert [s13.size, s2.size] == f["per_expert"]
    assert f["experts"] * (s13.size + s2.size) == f["total"]


def test_weight_block_invariants_ragged():
    w = _bf16_data((300, 200), 11, scale=0.05)
    q, s = quant.quant_weight_block(w)
    assert s.shape == (3, 2)
    for i in range(3):
        for j in range(2):
            blk = q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert np.abs(e4m3.decode(blk)).max() == 448.0
            # each block equals the per-tensor quantization of that block alone
            qt, st = quant.quant_tensor(w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128])
            np.testing.assert_array_equal(blk, qt)
            assert s[i, j] == st


def test_weight_block_vs_transposed_group_quant():
    # a 1 x 128 block grid on W is the group quantizer on W's rows
    w = _bf16_data((6, 384), 12)
    q1, s1 = quant.quant_weight_block(w, 1, 128)
    q2, s2 = quant.quant_group(w, 128)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)


def test_tensor_quant_is_single_block():
    w = _bf16_data((130, 260), 13)
    q1, s1 = quant.quant_tensor(w)
    q2, s2 = quant.quant_weight_block(w, 130, 260)
    np.testing.assert_array_equal(q1, q2)
    assert s2.shape == (1, 1) and s2[0, 0] == s1


# ------------------------------------------------------------------------ MXFP8

def _all_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    return bf16.to_f32(bits)


def test_mx_exponent_exhaustive_vs_frexp():
    a = _all_positive_bf16()
    e = quant.mx_exponent(a)
    a_eff = np.maximum(a, np.float32(1e-10)).astype(np.float64)
    # 448 = 1.75 * 2^8: with a = f * 2^E (f in [0.5, 1)), the smallest e with
    # a <= 448 * 2^e is E - 9, plus one when f > 0.875
    ref = np.array([math.frexp(v)[1] - 9 + (math.frexp(v)[0] > 0.875) for v in a_eff])
    np.testing.assert_array_equal(e, ref)


def test_mx_exponent_no_overflow_and_tight():
    a = np.maximum(_all_positive_bf16(), np.float32(1e-10)).astype(np.float64)
    e = quant.mx_exponent(a)
    t = np.ldexp(a, -e)
    assert np.all(t <= 448.0) and np.all(t > 224.0)


def test_mx_byte_range_within_ue8m0():
    f = GOLDEN["ue8m0_range_log2"]
    e = quant.mx_exponent(_all_positive_bf16())
    assert e.min() >= f["min"] and e.max() <= f["max"]
    assert (e + 127).max() <= 254                      # 255 is never produced


def test_mx_quant_block_max_and_overhead():
    f = GOLDEN["mx_block"]
    x = _bf16_data((16, 512), 14, outlier_cols=(9,))
    q, sb = quant.quant_mx(x, f["block_k"])
    assert sb.shape == (16, 512 // 32) and sb.dtype == np.uint8
    blockmax = np.abs(e4m3.decode(q)).reshape(16, 16, 32).max(axis=2)
    assert np.all(blockmax >= 224) and np.all(blockmax <= 448)
    assert sb.nbytes / q.nbytes == GOLDEN["scale_overhead"]["group128"]
    # dequantized error bound (power-of-two scale: no fp32 division rounding)
    S = np.ldexp(1.0, np.repeat(sb.astype(np.int64) - 127, 32, axis=1))
    dq = e4m3.decode(q) * S
    ratio = np.abs(x) / S
    n = ratio >= 2.0 ** -6
    assert np.all(np.abs(dq - x)[n] <= 2.0 ** -4 * np.abs(x[n]))


def test_mx_power_of_two_equivariance():
    x = _bf16_data((8, 256), 15)
    q0, b0 = quant.quant_mx(x)
    q1, b1 = quant.quant_mx(np.ldexp(x, 7))
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(b1.astype(int), b0.astype(int) + 7)
