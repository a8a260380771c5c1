"""Planted mistakes in the oracle (CPU only): each plausible slip must fail a pin.

Every case patches one oracle function with a subtly wrong variant and runs
the relevant pin check; the check has to raise.  Nothing here touches a GPU.
"""
import math

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm, quant
from tests.exact_arith import rn32_quotient


def _encode_ties_away(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    pos = e4m3.DECODE_TABLE[:127]
    lo = np.clip(np.searchsorted(pos, a, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    mid = (pos[lo] + pos[hi]) / 2
    code = np.where(a < mid, lo, hi)                 # ties go up: wrong
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def _encode_truncate(v):
    v = np.asarray(v, np.float64)
    pos = e4m3.DECODE_TABLE[:127]
    lo = np.clip(np.searchsorted(pos, np.abs(v), side="right") - 1, 0, 126)
    return (lo | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def _check_encode_vs_torch(enc):
    rng = np.random.default_rng(0)
    vals = np.clip(rng.uniform(-448, 448, 50_000).astype(np.float32), -448, 448)
    pos = e4m3.DECODE_TABLE[:127]
    vals = np.concatenate([vals, ((pos[:-1] + pos[1:]) / 2).astype(np.float32)])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(enc(vals), ref)


@pytest.mark.parametrize("bad", [_encode_ties_away, _encode_truncate])
def test_encoder_mistakes_are_caught(bad):
    _check_encode_vs_torch(e4m3.encode)          # the real one passes
    with pytest.raises(AssertionError):
        _check_encode_vs_torch(bad)


def _check_group_invariants(qfun):
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal((32, 512)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    q, s = qfun(x)
    dq = np.abs(e4m3.decode(q)).reshape(32, 4, 128).max(axis=2)
    assert np.all(dq == 448.0)
    amax = np.abs(x).reshape(32, 4, 128).max(axis=2)
    np.testing.assert_array_equal(np.asarray(s, np.float64), rn32_quotient(amax, np.float32(448.0)))
    # equivariance under powers of two
    q2, s2 = qfun(np.ldexp(x, 3))
    np.testing.assert_array_equal(q2, q)


def _group_scale_wrong_constant(x):
    x = np.asarray(x, np.float32)
    s = (np.abs(x).reshape(x.shape[0], -1, 128).max(axis=2) / np.float32(240)).astype(np.float32)
    return quant.quantize_with_scale(x, np.repeat(s, 128, axis=1)), s


def _group_off_by_one_group(x):
    q, s = quant.quant_group(x)
    return q, np.roll(s, 1, axis=1)


@pytest.mark.parametrize("bad", [_group_scale_wrong_constant, _group_off_by_one_group])
def test_group_quant_mistakes_are_caught(bad):
    _check_group_invariants(quant.quant_group)
    with pytest.raises(AssertionError):
        _check_group_invariants(bad)


def _check_gemm(gfun):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 384)).astype(np.float32)
    w = (rng.standard_normal((260, 384)) / 20).astype(np.float32)
    qa, sa = quant.quant_group(x)
    qw, sw = quant.quant_weight_block(w)
    _, acc = gfun(qa, sa, qw, sw)
    np.testing.assert_allclose(acc, gemm.gemm_dequant_reference(qa, sa, qw, sw), rtol=1e-12)


def _gemm_transposed_wscale(qa, sa, qw, sw):
    # uses the weight-scale grid of block (b, j//128) instead of (j//128, b)
    sw_t = np.resize(np.asarray(sw).T, np.asarray(sw).shape)
    return gemm.gemm_blockscale(qa, sa, qw, sw_t)


def _gemm_drop_last_block(qa, sa, qw, sw):
    qa = qa.copy()
    qa[:, 256:] = 0
    return gemm.gemm_blockscale(qa, sa, qw, sw)


def _gemm_scales_outside_sum(qa, sa, qw, sw):
    A, W = e4m3.decode(qa), e4m3.decode(qw)
    acc = (A @ W.T) * sa.mean(axis=1)[:, None] * np.repeat(sw.mean(axis=1), 128)[None, :W.shape[0]]
    return None, acc


@pytest.mark.parametrize("bad", [_gemm_transposed_wscale, _gemm_drop_last_block,
                                 _gemm_scales_outside_sum])
def test_gemm_mistakes_are_caught(bad):
    _check_gemm(gemm.gemm_blockscale)
    with pytest.raises(AssertionError):
        _check_gemm(bad)


def _check_mx_exponent(efun):
    a = np.ldexp(np.linspace(1, 2, 4097)[:-1], 3).astype(np.float32)
    e = efun(a)
    t = np.ldexp(a.astype(np.float64), -e)
    assert np.all(t <= 448) and np.all(t > 224)


def _mx_exponent_round_nearest(amax):
    a = np.maximum(np.asarray(amax, np.float32), np.float32(1e-10)).astype(np.float64)
    return np.rint(np.log2(a / 448.0)).astype(np.int64)


def _mx_exponent_floor(amax):
    a = np.maximum(np.asarray(amax, np.float32), np.float32(1e-10)).astype(np.float64)
    return np.floor(np.log2(a / 448.0)).astype(np.int64)


@pytest.mark.parametrize("bad", [_mx_exponent_round_nearest, _mx_exponent_floor])
def test_mx_exponent_mistakes_are_caught(bad):
    _check_mx_exponent(quant.mx_exponent)
    with pytest.raises(AssertionError):
        _check_mx_exponent(bad)


def test_rmsnorm_missing_eps_or_sqrt_is_caught():
    K = 64
    c = np.float32(0.001)
    x = np.full((1, K), c, np.float32)
    r, _, _ = quant.rms_inv(x, 1e-6)
    expect = np.float32(1.0 / math.sqrt(float(c) ** 2 + float(np.float32(1e-6))))
    assert r[0] == expect
    assert np.float32(1.0 / math.sqrt(float(c) ** 2)) != expect       # eps dropped
    assert np.float32(1.0 / (float(c) ** 2 + 1e-6)) != expect          # sqrt dropped


# ------------------------------------------------------------ residual add

def _add_wrong_sign(x, h):
    from oracle import bf16
    return bf16.round_from_f64(np.asarray(x, np.float64) - np.asarray(h, np.float64))


def _add_truncating(x, h):
    s = (np.asarray(x, np.float64) + np.asarray(h, np.float64)).astype(np.float32)
    return (s.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@pytest.mark.parametrize("bad", [_add_wrong_sign, _add_truncating])
def test_residual_add_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_residual as pins
    monkeypatch.setattr(quant, "residual_add", bad)
    with pytest.raises(AssertionError):
        pins.test_residual_add_is_correctly_rounded()


def _norm_of_unrounded_sum(x, h, g, eps, static_scale=None, group=128, r=None):
    from oracle import bf16
    z = quant.residual_add(x, h)
    exact = (np.asarray(x, np.float64) + np.asarray(h, np.float64)).astype(np.float32)
    r, r_alt, amb = quant.rms_inv(exact, eps)
    y = quant.rmsnorm_apply(exact, g, r)
    q, s = quant.quant_group(bf16.to_f32(y), group)
    return {"z": z, "q": q, "s": s, "y": y, "r": r, "r_alt": r_alt, "ambiguous": amb}


def _norm_of_stream_before_add(x, h, g, eps, static_scale=None, group=128, r=None):
    out = quant.rmsnorm_quant(np.asarray(x, np.float32), g, eps)
    out["z"] = quant.residual_add(x, h)
    return out


@pytest.mark.parametrize("bad", [_norm_of_unrounded_sum, _norm_of_stream_before_add])
def test_fused_norm_input_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_residual as pins
    monkeypatch.setattr(quant, "add_rmsnorm_quant", bad)
    caught = 0
    for pin in (pins.test_constant_sum_rows_closed_form, pins.test_symmetric_in_stream_and_sublayer_output,
                pins.test_norm_reads_the_stored_stream):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1


# ------------------------------------------------------ power-of-two scales

def _requant_floor_exponent(q, s, block_n=128, block_k=128):
    from oracle import e4m3
    q = np.asarray(q, np.uint8)
    N, K = q.shape
    e = np.floor(np.log2(np.asarray(s, np.float64))).astype(np.int64)     # rounds down
    s2 = quant.pow2_scale(e)
    m = np.repeat(np.repeat(np.asarray(s, np.float64) / s2, block_n, 0), block_k, 1)[:N, :K]
    return e4m3.encode(np.clip(e4m3.decode(q) * m, -448.0, 448.0)), s2


def _requant_truncating(q, s, block_n=128, block_k=128):
    from oracle import e4m3
    q = np.asarray(q, np.uint8)
    N, K = q.shape
    f, k = np.frexp(np.asarray(s, np.float64))
    s2 = quant.pow2_scale(np.where(f == 0.5, k - 1, k))
    m = np.repeat(np.repeat(np.asarray(s, np.float64) / s2, block_n, 0), block_k, 1)[:N, :K]
    v = e4m3.decode(q) * m
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -9)))
    step = np.exp2(np.maximum(e, -6) - 3)
    return e4m3.encode(np.clip(np.trunc(v / step) * step, -448.0, 448.0)), s2     # drops the rounding


@pytest.mark.parametrize("bad", [_requant_floor_exponent, _requant_truncating])
def test_requant_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_pow2 as pins
    monkeypatch.setattr(quant, "requant_weight_pow2", bad)
    with pytest.raises(AssertionError):
        pins.test_requant_every_code_against_exact_rounding()


def _group_pow2_nearest_exponent(x, group=128):
    x = np.asarray(x, np.float32)
    M, K = x.shape
    G = -(-K // group)
    from oracle import e4m3
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, G), np.float32)
    for g in range(G):
        cols = slice(g * group, min(K, (g + 1) * group))
        amax = np.maximum(np.max(np.abs(x[:, cols]), axis=1), np.float32(1e-10)).astype(np.float64)
        e = np.round(np.log2(amax / 448.0)).astype(np.int64)
        s[:, g] = quant.pow2_scale(e)
        q[:, cols] = e4m3.encode(np.clip(np.ldexp(x[:, cols].astype(np.float64), -e[:, None]), -448, 448))
    return q, s


def test_group_pow2_mistake_is_caught(monkeypatch):
    import tests.test_oracle_pow2 as pins
    monkeypatch.setattr(quant, "quant_group_pow2", _group_pow2_nearest_exponent)
    with pytest.raises(AssertionError):
        pins.test_group_pow2_scales_bracket_amax()


# ------------------------------------------------------------------ MoE

def _sharded_as_one_grid(w, shard):
    return quant.quant_weight_block(w)


def test_shard_rule_mistake_is_caught(monkeypatch):
    import tests.test_oracle_moe as pins
    monkeypatch.setattr(quant, "quant_weight_block_sharded", _sharded_as_one_grid)
    with pytest.raises(AssertionError):
        pins.test_shard_rule_when_intermediate_is_not_a_multiple_of_128()


def test_grouped_offset_mistake_is_caught(monkeypatch):
    import tests.test_oracle_moe as pins
    real = gemm.gemm_grouped_blockscale

    def shifted(qa, sa, qw, sw, offsets, shard=0, rows=None):
        off = np.asarray(offsets).copy()
        off[1:-1] += 1                                        # rows slip into the next expert
        return real(qa, sa, qw, sw, off, shard=shard, rows=rows)

    monkeypatch.setattr(gemm, "gemm_grouped_blockscale", shifted)
    with pytest.raises(AssertionError):
        pins.test_grouped_gemm_against_per_expert_dequantized_products(0)


# ------------------------------------------- the two quotients of the quantizer

def _group_scale_reciprocal(amax):
    # amax * RN32(1/448) instead of the division amax / 448
    a = np.maximum(np.asarray(amax, np.float32), np.float32(1e-10))
    return (a * (np.float32(1) / np.float32(448))).astype(np.float32)


def _quantize_reciprocal(x, s):
    # x * RN32(1/s) instead of the division x / s
    x = np.asarray(x, np.float32)
    s = np.asarray(s, np.float32)
    t = (x * (np.float32(1) / s).astype(np.float32)).astype(np.float32)
    return e4m3.encode(np.clip(t, -448, 448))


def test_group_scale_reciprocal_is_caught():
    from tests.test_oracle_exact import check_group_scale
    check_group_scale(quant.group_scale)
    with pytest.raises(AssertionError):
        check_group_scale(_group_scale_reciprocal)


def test_quantize_reciprocal_is_caught():
    from tests.test_oracle_exact import check_quantize_with_scale
    check_quantize_with_scale(quant.quantize_with_scale)
    with pytest.raises(AssertionError):
        check_quantize_with_scale(_quantize_reciprocal)
