"""Pins of the oracle's fused RMSNorm front end and scaled GEMMs (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, gemm, quant


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


# ------------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_closed_form():
    K, eps = 256, 1e-6
    c = np.float32(0.8125)                        # exactly bf16
    x = np.full((1, K), c, np.float32)
    g = np.ones(K, np.float32)
    y, r, _, amb = quant.rmsnorm(x, g, eps)
    expect_r = np.float32(1.0 / math.sqrt(float(c) ** 2 + float(np.float32(eps))))
    assert r[0] == expect_r and not amb[0]
    yv = bf16.to_f64(y)
    assert np.all(yv == yv[0, 0])
    assert abs(yv[0, 0] - 1.0) <= 2.0 ** -8


def test_rmsnorm_vs_torch_rms_norm_fp64():
    rng = np.random.default_rng(0)
    x = _bf16(rng.standard_normal((64, 1536)) * 3)
    x[:, 17] *= 50
    x = _bf16(x)
    g = _bf16(rng.uniform(0.5, 1.5, 1536))
    y, _, _, _ = quant.rmsnorm(x, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (1536,),
                                       torch.from_numpy(g.astype(np.float64)), eps=float(np.float32(1e-6)))
    ref = ref.numpy()
    yv = bf16.to_f64(y)
    # one bf16 rounding (half an ulp: at most 2^-8 relative) plus fp32 roundings
    assert np.all(np.abs(yv - ref) <= np.abs(ref) * (2.0 ** -8 + 2.0 ** -21) + 1e-30)


def test_rmsnorm_unit_gain_gives_unit_mean_square():
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal((32, 2048)) * 0.5)
    y, _, _, _ = quant.rmsnorm(x, np.ones(2048, np.float32), 1e-6)
    ms = np.mean(bf16.to_f64(y) ** 2, axis=1)
    np.testing.assert_allclose(ms, 1.0, rtol=5e-3)


def test_rmsnorm_quant_is_norm_then_group_quant():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((16, 640)))
    g = _bf16(rng.uniform(0.5, 1.5, 640))
    out = quant.rmsnorm_quant(x, g, 1e-6)
    y, _, _, _ = quant.rmsnorm(x, g, 1e-6)
    q, s = quant.quant_group(bf16.to_f32(y))
    np.testing.assert_array_equal(out["y"], y)
    np.testing.assert_array_equal(out["q"], q)
    np.testing.assert_array_equal(out["s"], s)


def test_rms_inv_neighbour_is_adjacent_fp32():
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((200, 512)))
    r, r_alt, amb = quant.rms_inv(x, 1e-6)
    assert np.all(np.abs(np.nextafter(r, r_alt) - r_alt) == 0)
    assert amb.sum() <= 2          # near-ties are rare (rate about 2^-16 per row)


# ---------------------------------------------------------------------- GEMMs

def _quantized_problem(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((N, K)) / math.sqrt(K))
    qa, sa = quant.quant_group(x)
    qw, sw = quant.quant_weight_block(w)
    return x, w, qa, sa, qw, sw


@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (5, 300, 520), (33, 130, 128)])
def test_block_gemm_equals_dequantized_matmul(M, N, K):
    _, _, qa, sa, qw, sw = _quantized_problem(M, N, K, M + N + K)
    y, acc = gemm.gemm_blockscale(qa, sa, qw, sw)
    ref = gemm.gemm_dequant_reference(qa, sa, qw, sw)
    np.testing.assert_allclose(acc, ref, rtol=1e-12, atol=1e-300)
    assert y.shape == (M, N) and y.dtype == np.uint16


def test_block_gemm_exhaustive_code_products():
    # one non-zero per row, unit scales: Y[i, j] = dec(a_i) * dec(w_j), and
    # every such product is exact in bf16 (8 significant bits)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n = codes.size
    qa = np.zeros((n, 128), np.uint8)
    qa[:, 0] = codes
    qw = np.zeros((n, 128), np.uint8)
    qw[:, 0] = codes
    sa = np.ones((n, 1), np.float32)
    sw = np.ones((-(-n // 128), 1), np.float32)
    y, _ = gemm.gemm_blockscale(qa, sa, qw, sw)
    v = e4m3.DECODE_TABLE[codes]
    outer = torch.from_numpy(np.outer(v, v).astype(np.float32)).to(torch.bfloat16)
    # values compared (a sum of products is +0 where the outer product has -0)
    np.testing.assert_array_equal(bf16.to_f64(y), outer.to(torch.float64).numpy())


def test_block_gemm_scale_locality():
    _, _, qa, sa, qw, sw = _quantized_problem(8, 256, 384, 7)
    _, acc0 = gemm.gemm_blockscale(qa, sa, qw, sw)
    sa2 = sa.copy()
    sa2[3, :] *= 2                                  # row 3 of the activations
    _, acc1 = gemm.gemm_blockscale(qa, sa2, qw, sw)
    np.testing.assert_array_equal(acc1[3], 2 * acc0[3])
    np.testing.assert_array_equal(np.delete(acc1, 3, 0), np.delete(acc0, 3, 0))
    sw2 = sw.copy()
    sw2[1, :] *= 4                                  # second 128-row block of W
    _, acc2 = gemm.gemm_blockscale(qa, sa, qw, sw2)
    np.testing.assert_array_equal(acc2[:, 128:], 4 * acc0[:, 128:])
    np.testing.assert_array_equal(acc2[:, :128], acc0[:, :128])
    sa3 = sa.copy()
    sa3[:, 1] = 0                                   # drop K block 1 only
    _, acc3 = gemm.gemm_blockscale(qa, sa3, qw, sw)
    keep = np.ones(384, bool)
    keep[128:256] = False
    ref = gemm.gemm_dequant_reference(qa * keep, sa, qw, sw)
    np.testing.assert_allclose(acc3, ref, rtol=1e-12)


def test_block_gemm_bias_added_before_rounding():
    _, _, qa, sa, qw, sw = _quantized_problem(4, 128, 256, 8)
    bias = _bf16(np.linspace(-2, 2, 128)).astype(np.float64)
    y, acc = gemm.gemm_blockscale(qa, sa, qw, sw, bias=bias)
    _, acc0 = gemm.gemm_blockscale(qa, sa, qw, sw)
    np.testing.assert_allclose(acc, acc0 + bias[None, :], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(y, bf16.round_from_f64(acc0 + bias[None, :]))


def test_block_gemm_close_to_unquantized():
    # the debugging check the pages suggest: FP8 result vs the high-precision one
    x, w, qa, sa, qw, sw = _quantized_problem(32, 256, 1024, 9)
    y, _ = gemm.gemm_blockscale(qa, sa, qw, sw)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    err = np.abs(bf16.to_f64(y) - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert err.max() < 0.05


def test_pertensor_equals_block_with_uniform_scales():
    rng = np.random.default_rng(10)
    x = _bf16(rng.standard_normal((12, 384)))
    w = _bf16(rng.standard_normal((200, 384)) * 0.1)
    sx = np.float32(np.abs(x).max() / np.float32(448))
    qa = quant.quant_static(x, sx)
    qw, sw = quant.quant_tensor(w)
    y1, acc1 = gemm.gemm_pertensor(qa, sx, qw, sw)
    sa = np.full((12, 3), sx, np.float32)
    swb = np.full((2, 3), sw, np.float32)
    _, acc2 = gemm.gemm_blockscale(qa, sa, qw, swb)
    np.testing.assert_allclose(acc1, acc2, rtol=1e-13)
    # and scalar scales leave the sum: acc == (sum of code products) * sx * sw
    raw = e4m3.decode(qa) @ e4m3.decode(qw).T
    np.testing.assert_array_equal(acc1, raw * float(sx) * float(sw))


def test_pertensor_vs_torch_scaled_mm_semantics():
    # torch's CPU reference for a scalar-scaled fp8 matmul: dequantize, matmul
    rng = np.random.default_rng(11)
    x = _bf16(rng.standard_normal((8, 256)))
    w = _bf16(rng.standard_normal((64, 256)))
    qa, sx = quant.quant_tensor(x)
    qw, sw = quant.quant_tensor(w)
    ta = torch.from_numpy(qa).view(torch.float8_e4m3fn).to(torch.float64) * float(sx)
    tw = torch.from_numpy(qw).view(torch.float8_e4m3fn).to(torch.float64) * float(sw)
    ref = (ta @ tw.T).numpy()
    _, acc = gemm.gemm_pertensor(qa, sx, qw, sw)
    np.testing.assert_allclose(acc, ref, rtol=1e-13)


def test_mx_gemm_equals_dequantized_matmul():
    rng = np.random.default_rng(12)
    x = _bf16(rng.standard_normal((9, 320)))
    w = _bf16(rng.standard_normal((70, 320)))
    qa, ea = quant.quant_mx(x)
    qw, ew = quant.quant_mx(w)
    y, acc = gemm.gemm_mx(qa, ea, qw, ew)
    ref = gemm.gemm_mx_dequant_reference(qa, ea, qw, ew)
    np.testing.assert_allclose(acc, ref, rtol=1e-12)
    ref_hp = x.astype(np.float64) @ w.astype(np.float64).T
    err = np.abs(bf16.to_f64(y) - ref_hp).max(axis=1) / np.abs(ref_hp).max(axis=1)
    assert err.max() < 0.06


def test_mx_gemm_exponent_add():
    # UE8M0: multiplying by a scale is adding exponents; bumping every block
    # byte of one operand row by 3 multiplies that row of Y by 8 exactly
    rng = np.random.default_rng(13)
    x = _bf16(rng.standard_normal((4, 128)))
    w = _bf16(rng.standard_normal((32, 128)))
    qa, ea = quant.quant_mx(x)
    qw, ew = quant.quant_mx(w)
    _, acc0 = gemm.gemm_mx(qa, ea, qw, ew)
    ea2 = ea.copy()
    ea2[2] += 3
    _, acc1 = gemm.gemm_mx(qa, ea2, qw, ew)
    np.testing.assert_array_equal(acc1[2], 8 * acc0[2])


def test_rows_subset_matches_full():
    _, _, qa, sa, qw, sw = _quantized_problem(20, 128, 256, 14)
    y, _ = gemm.gemm_blockscale(qa, sa, qw, sw)
    ys, _ = gemm.gemm_blockscale(qa, sa, qw, sw, rows=np.array([0, 7, 19]))
    np.testing.assert_array_equal(ys, y[[0, 7, 19]])
