"""GPU parity of the decode GEMM path (M <= 64, K % 128 == 0).

The decode kernel streams weights through per-wave LDS rings; its
configuration (six or two 16-column tiles per workgroup, ring depth) depends
on N and the CU count, so fp8q_set_plan_override (decode_wide) pins each
one here.  Shapes cover every row-tile count (M 1..64),
fewer K blocks than waves (K = 128, 384), ragged N (columns past the end of
the last tile) and both activation-scale layouts, in block, per-tensor and
MX scale modes.  Expected values come from the oracle; the tolerance is the
method's per-row bound.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import bf16 as obf16
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_helpers import CANARY_BF16, bf16_bits, bf16_host, canary_intact, check_gemm_rows, log, padded

pytestmark = pytest.mark.gpu

REL = 1e-2
SHAPES = [(1, 200, 128), (8, 1000, 384), (16, 520, 1024), (31, 296, 2048), (48, 1536, 640), (64, 776, 6144)]


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _dev_u8(a: np.ndarray, k: int) -> torch.Tensor:
    rows = a.shape[0]
    ld = -(-k // 16) * 16 + 16          # a padded leading dimension
    buf = torch.zeros(rows, ld, dtype=torch.uint8, device="cuda")
    buf[:, :k] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return buf[:, :k]


def _operands(M, N, K, seed):
    x = bf16_host(workloads.activations(M, K, seed, 0.01))
    w = bf16_host(workloads.weights(N, K, seed + 1))
    return x, w


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("wide", [0, 1])
@pytest.mark.parametrize("a_layout", [0, 1])
def test_decode_blockscale(plan, M, N, K, wide, a_layout):
    log(f"decode block M={M} N={N} K={K} wide={wide} layout={a_layout}")
    plan(decode_wide=wide)
    m = fq()
    x, w = _operands(M, N, K, 90 + M)
    qa, sa = oq.quant_group(x)
    qw, sw = oq.quant_weight_block(w)
    bias = obf16.to_f64(obf16.round_from_f64(np.linspace(-1.0, 1.0, N)))
    b_d = torch.from_numpy(bias.astype(np.float32)).to(torch.bfloat16).cuda()
    sa_d = torch.from_numpy(np.ascontiguousarray(sa.T if a_layout else sa)).cuda()
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_blockscale(_dev_u8(qa, K), sa_d, a_layout, _dev_u8(qw, K), torch.from_numpy(sw).cuda(), b_d, y,
                           m.GRAN_BLOCK128)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16), "y written outside [M, N]"
    yr, _ = og.gemm_blockscale(qa, sa, qw, sw, bias=bias)
    check_gemm_rows(bf16_bits(y), yr, f"decode block M={M} N={N} K={K} wide={wide}", REL)


@pytest.mark.parametrize("M,N,K", SHAPES[:4])
@pytest.mark.parametrize("wide", [0, 1])
def test_decode_pertensor(plan, M, N, K, wide):
    log(f"decode per-tensor M={M} N={N} K={K} wide={wide}")
    plan(decode_wide=wide)
    m = fq()
    x, w = _operands(M, N, K, 120 + M)
    sx = np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))
    qa = oq.quant_static(x, sx)
    qw, sw = oq.quant_tensor(w)
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_blockscale(_dev_u8(qa, K), torch.tensor([sx], device="cuda"), 0, _dev_u8(qw, K),
                           torch.tensor([sw], dtype=torch.float32, device="cuda"), None, y, m.GRAN_PER_TENSOR)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_pertensor(qa, sx, qw, sw)
    check_gemm_rows(bf16_bits(y), yr, f"decode per-tensor M={M} wide={wide}", REL)


@pytest.mark.parametrize("M,N,K", SHAPES[1:])
@pytest.mark.parametrize("wide", [0, 1])
def test_decode_mxfp8(plan, M, N, K, wide):
    log(f"decode mx M={M} N={N} K={K} wide={wide}")
    plan(decode_wide=wide)
    m = fq()
    x, w = _operands(M, N, K, 150 + M)
    qa, ea = oq.quant_mx(x)
    qw, ew = oq.quant_mx(w)
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_mxfp8(_dev_u8(qa, K), torch.from_numpy(ea).cuda(), _dev_u8(qw, K), torch.from_numpy(ew).cuda(),
                      None, y)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_mx(qa, ea, qw, ew)
    check_gemm_rows(bf16_bits(y), yr, f"decode mx M={M} wide={wide}", REL)


def test_decode_deterministic(plan):
    # fixed-order reduction of the waves' partial sums: identical bits twice
    plan(decode_wide=1)
    m = fq()
    M, N, K = 32, 1536, 6144
    x, w = _operands(M, N, K, 181)
    qa, sa = oq.quant_group(x)
    qw, sw = oq.quant_weight_block(w)
    args = (_dev_u8(qa, K), torch.from_numpy(sa).cuda(), _dev_u8(qw, K), torch.from_numpy(sw).cuda())
    y1 = bf16_bits(m.gemm_blockscale(*args))
    y2 = bf16_bits(m.gemm_blockscale(*args))
    np.testing.assert_array_equal(y1, y2)
