"""Pins of the oracle's power-of-two ("block FP8 as MXFP8") quantizers and of
the scaled GEMM on such scales (CPU only).

Independent checks: the power-of-two bracket of every scale around amax/448,
closed forms where amax/448 is itself a power of two (then the fp32-scale
quantizers, pinned elsewhere, must agree exactly), a brute-force
re-quantization of every E4M3 code against exact rational rounding, the
exponent-add form of the GEMM (the MX GEMM with 128-wide blocks) against the
fp32-multiply form, and the size of the accuracy cost against the fp32
scales.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, gemm, quant


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _is_pow2(s):
    f, _ = np.frexp(np.asarray(s, np.float64))
    return np.all(f == 0.5)


def _acts(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, max(1, K // 1000), replace=False)] *= 50
    return _bf16(x)


def test_group_pow2_scales_bracket_amax():
    x = _acts(64, 1000, 0)
    x[3] = 0.0
    x[4, :128] = 448.0 * 2.0 ** -5                    # amax/448 exactly a power of two
    q, s = quant.quant_group_pow2(x)
    assert s.shape == (64, 8) and _is_pow2(s)
    for g in range(8):
        cols = slice(128 * g, min(1000, 128 * g + 128))
        amax = np.maximum(np.max(np.abs(x[:, cols]), axis=1).astype(np.float64), float(np.float32(1e-10)))
        sg = s[:, g].astype(np.float64)
        assert np.all(amax <= 448.0 * sg) and np.all(amax > 224.0 * sg)
        top = np.max(np.abs(e4m3.decode(q[:, cols])), axis=1)
        nz = amax > float(np.float32(1e-10))
        assert np.all(top[nz] > 224.0 * 0.93) and np.all(top <= 448.0)
    assert s[4, 0] == np.float32(2.0 ** -5) and np.max(q[4, :128] & 0x7F) == 0x7E
    assert np.all(q[3] == 0)


def test_group_pow2_equals_fp32_path_when_scale_is_pow2():
    # rows whose every group max is 448 * 2^k: both rules give s = 2^k
    rng = np.random.default_rng(1)
    K = 512
    x = _bf16(rng.uniform(-1, 1, (16, K)))
    k = rng.integers(-8, 8, (16, K // 128))
    for g in range(K // 128):
        x[:, 128 * g] = 448.0 * np.exp2(k[:, g])
        x[:, 128 * g + 1:128 * (g + 1)] *= 448.0 * np.exp2(k[:, g])[:, None]
    x = _bf16(x)
    q1, s1 = quant.quant_group_pow2(x)
    q2, s2 = quant.quant_group(x)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(q1, q2)


def test_group_pow2_dequant_error_bound():
    x = _acts(32, 768, 2)
    q, s = quant.quant_group_pow2(x)
    xr = e4m3.decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    # half an E4M3 ulp (2^-4 relative) for normal codes, half the subnormal step below
    tol = np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(s.astype(np.float64), 128, axis=1) * 2.0 ** -10)
    assert np.all(np.abs(xr - x) <= tol)


def test_weight_pow2_blocks():
    rng = np.random.default_rng(3)
    w = _bf16(rng.standard_normal((300, 260)) / 16)
    w[:128, :128] *= 448.0 * 2.0 ** -9 / np.max(np.abs(w[:128, :128]))
    w = _bf16(w)
    q, s = quant.quant_weight_block_pow2(w)
    assert s.shape == (3, 3) and _is_pow2(s)
    for i in range(3):
        for j in range(3):
            blk = w[128 * i:128 * i + 128, 128 * j:128 * j + 128].astype(np.float64)
            amax = np.max(np.abs(blk))
            assert 224.0 * s[i, j] < amax <= 448.0 * s[i, j]
    qf, sf = quant.quant_weight_block(w)
    if sf[0, 0] == s[0, 0]:                            # amax/448 a power of two
        np.testing.assert_array_equal(q[:128, :128], qf[:128, :128])


def _nearest_e4m3_exact(v: Fraction) -> int:
    """Code of the E4M3 value nearest to v (ties to the even code), by
    enumerating every finite code: independent of the oracle's encoder.
    A value that rounds to zero keeps its sign (0x80 for negatives)."""
    best = None
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        d = abs(Fraction(e4m3.decode_code(c)) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    code = best[1]
    if code & 0x7F == 0:
        return 0x80 if v < 0 else 0x00
    return code


def test_requant_every_code_against_exact_rounding():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    N = len(codes)
    for sv in (0.00842026, 0.75, 0.5, 3.0e-5, 1.0 / 3.0):
        s = np.full((1, 1), np.float32(sv), np.float32)
        q = np.tile(codes[:, None], (1, 4))            # [254, 4]: one block
        s_blocks = np.full((-(-N // 128), 1), np.float32(sv), np.float32)
        q2, s2 = quant.requant_weight_pow2(q, s_blocks)
        e = math.ceil(math.log2(float(s[0, 0])))
        if Fraction(float(s[0, 0])) <= Fraction(2) ** (e - 1):
            e -= 1
        assert np.all(s2 == np.float32(2.0 ** e))
        m = Fraction(float(np.float32(sv))) / Fraction(2) ** e
        for r, c in enumerate(codes):
            v = Fraction(e4m3.decode_code(int(c))) * m
            expect = _nearest_e4m3_exact(v)
            got = int(q2[r, 0])
            if v == 0:
                assert got & 0x7F == 0 and (got >> 7) == (c >> 7)
            else:
                assert got == expect, (sv, c, got, expect)


def test_requant_identity_on_pow2_scales():
    rng = np.random.default_rng(4)
    w = _bf16(rng.standard_normal((256, 384)))
    q, s = quant.quant_weight_block_pow2(w)
    q2, s2 = quant.requant_weight_pow2(q, s)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s)


def test_pow2_gemm_is_exponent_add_gemm():
    # the fp32-multiply formula on power-of-two scales equals the MX
    # (exponent-add) formula with 128-wide blocks and expanded weight scales
    x = _acts(24, 640, 5)
    rng = np.random.default_rng(6)
    w = _bf16(rng.standard_normal((300, 640)) / math.sqrt(640))
    qa, sa = quant.quant_group_pow2(x)
    qw, sw = quant.quant_weight_block_pow2(w)
    y1, _ = gemm.gemm_blockscale(qa, sa, qw, sw)
    ea = (np.frexp(sa.astype(np.float64))[1] - 1 + 127).astype(np.uint8)
    ew = (np.frexp(sw.astype(np.float64))[1] - 1 + 127).astype(np.uint8)
    ew_rows = np.repeat(ew, 128, axis=0)[:300]
    y2, _ = gemm.gemm_mx(qa, ea, qw, ew_rows, block=128)
    np.testing.assert_array_equal(y1, y2)


def test_pow2_accuracy_cost_vs_fp32_scales():
    # the cost the pages name: power-of-two scales quantize a little more
    # coarsely.  Relative error of the layer output against the unquantized
    # fp64 product: larger than with fp32 scales, but by less than 2x.
    x = _acts(128, 2048, 7)
    rng = np.random.default_rng(8)
    w = _bf16(rng.standard_normal((512, 2048)) / math.sqrt(2048))
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    qa, sa = quant.quant_group(x)
    qw, sw = quant.quant_weight_block(w)
    y32 = bf16.to_f64(gemm.gemm_blockscale(qa, sa, qw, sw)[0])
    qa2, sa2 = quant.quant_group_pow2(x)
    qw2, sw2 = quant.requant_weight_pow2(qw, sw)
    y2 = bf16.to_f64(gemm.gemm_blockscale(qa2, sa2, qw2, sw2)[0])
    e32 = np.linalg.norm(y32 - exact) / np.linalg.norm(exact)
    e2 = np.linalg.norm(y2 - exact) / np.linalg.norm(exact)
    print(f"relative output error: fp32 scales {e32:.4%}, power-of-two scales {e2:.4%}")
    assert e32 < e2 < 2.0 * e32


def test_fused_norm_pow2_exit_is_norm_then_pow2_quant():
    # the pow2 exit of the fused front end quantizes the bf16 y (pinned
    # RMSNorm) with the power-of-two group quantizer pinned above
    rng = np.random.default_rng(9)
    x = _bf16(rng.standard_normal((8, 640)))
    h = _bf16(rng.standard_normal((8, 640)) / 4)
    g = _bf16(rng.uniform(0.5, 1.5, 640))
    out = quant.add_rmsnorm_quant(x, h, g, 1e-6, pow2=True)
    assert _is_pow2(out["s"])
    yv = bf16.to_f64(out["y"])
    for gi in range(5):
        cols = slice(128 * gi, 128 * gi + 128)
        amax = np.max(np.abs(yv[:, cols]), axis=1)
        assert np.all(amax <= 448.0 * out["s"][:, gi]) and np.all(amax > 224.0 * out["s"][:, gi])
    plain = quant.add_rmsnorm_quant(x, h, g, 1e-6)
    np.testing.assert_array_equal(out["y"], plain["y"])
    np.testing.assert_array_equal(out["z"], plain["z"])
