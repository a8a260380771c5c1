"""Pins of the oracle's MoE pieces (CPU only): stacked-shard weight scales
(the per-shard ceil rule the pages point out, and its scale count for the
pages' w13 example) and the grouped GEMM over expert-sorted rows, checked
against a second formulation (per-expert dequantized fp64 products with the
shards dequantized separately)."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, gemm, quant


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def test_w13_scale_count_of_the_pages_example():
    # H = 7168, I_p = 2048: 2 * 16 * 56 = 1792 scales per expert
    H, I = 7168, 2048
    _, s = quant.quant_weight_block_sharded(np.zeros((2 * I, H), np.float32), I)
    assert s.shape == (32, 56) and s.size == 1792


def test_shard_rule_when_intermediate_is_not_a_multiple_of_128():
    # I_p = 1088: each shard rounds up on its own -> 2 * 9 = 18 scale rows,
    # not ceil(2176 / 128) = 17; the gate's last block holds rows 1024..1087
    # only, the up shard's first block starts at row 1088
    I, K = 1088, 256
    w = np.ones((2 * I, K), np.float32)
    w[I:] = 100.0
    q, s = quant.quant_weight_block_sharded(w, I)
    assert s.shape == (18, 2)
    assert np.all(s[:9] == quant.group_scale(np.float32(1.0)))
    assert np.all(s[9:] == quant.group_scale(np.float32(100.0)))
    assert np.all(e4m3.decode(q[:I]) == 448.0) and np.all(e4m3.decode(q[I:]) == 448.0)
    rows = gemm.weight_scale_rows(2 * I, I)
    assert rows[1087] == 8 and rows[1088] == 9 and rows[-1] == 17
    # unsharded quantization mixes the shards in the straddling block
    _, s_plain = quant.quant_weight_block(w)
    assert s_plain.shape == (17, 2) and s_plain[8, 0] == quant.group_scale(np.float32(100.0))


def _moe_problem(counts, N, K, seed, shard=0):
    rng = np.random.default_rng(seed)
    M = int(sum(counts))
    x = _bf16(rng.standard_normal((M, K)))
    qa, sa = quant.quant_group(x)
    E = len(counts)
    ws = [_bf16(rng.standard_normal((N, K)) / math.sqrt(K)) for _ in range(E)]
    if shard:
        pairs = [quant.quant_weight_block_sharded(w, shard) for w in ws]
    else:
        pairs = [quant.quant_weight_block(w) for w in ws]
    qw = np.stack([p[0] for p in pairs])
    sw = np.stack([p[1] for p in pairs])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return qa, sa, qw, sw, offsets


def _dequant_sharded(q, s, shard):
    if not shard:
        return gemm.dequant_groups(q, s, 128, 128)
    nb = -(-shard // 128)
    parts = [gemm.dequant_groups(q[i:i + shard], s[(i // shard) * nb:(i // shard + 1) * nb], 128, 128)
             for i in range(0, q.shape[0], shard)]
    return np.concatenate(parts)


@pytest.mark.parametrize("shard", [0, 192])
def test_grouped_gemm_against_per_expert_dequantized_products(shard):
    counts = [0, 1, 37, 300, 0, 130]
    N, K = 384, 640
    qa, sa, qw, sw, off = _moe_problem(counts, N, K, 1 + shard, shard)
    y = bf16.to_f64(gemm.gemm_grouped_blockscale(qa, sa, qw, sw, off, shard=shard))
    Xd = gemm.dequant_groups(qa, sa, 1, 128)
    for e in range(len(counts)):
        r = slice(off[e], off[e + 1])
        ref = Xd[r] @ _dequant_sharded(qw[e], sw[e], shard).T
        # one bf16 rounding apart at most (the references sum in another order)
        assert np.all(np.abs(y[r] - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)


def test_grouped_gemm_rows_subset_and_expert_boundaries():
    counts = [5, 0, 64, 3]
    qa, sa, qw, sw, off = _moe_problem(counts, 256, 384, 7)
    full = gemm.gemm_grouped_blockscale(qa, sa, qw, sw, off)
    rows = np.array([0, 4, 5, 68, 71])            # first/last rows of experts 0, 2, 3
    np.testing.assert_array_equal(gemm.gemm_grouped_blockscale(qa, sa, qw, sw, off, rows=rows), full[rows])
    # a row multiplied by the wrong expert's weight would differ
    wrong, _ = gemm.gemm_blockscale(qa, sa, qw[3], sw[3], rows=[4])
    assert not np.array_equal(wrong[0], full[4])
