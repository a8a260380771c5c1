"""GPU parity of every tile plan of the prefill GEMM path.

The fast kernel has two tile configurations (256x256 and 128x128) and splits
the last, partly filled round of tiles into half-height tiles.  The plan
depends on the CU count; fp8q_set_plan_override (configuration, CU count
to plan for, tail split) pins it here so that
each configuration runs with and without split tiles on shapes the oracle
finishes quickly.  Ragged M and N put rows and columns past the ends inside
split tiles.  Expected values come from the oracle; the tolerance is the
method's per-row bound (see test_gpu_gemm).
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

# (cfg, slots, split): cfg 0 with 9 tiles on 6 CUs -> 3 tiles split; cfg 1
# with 25 tiles on 5 CUs (10 slots) -> 5 split; and both without splitting
PLANS = [(0, 6, 1), (0, 6, 0), (1, 5, 1), (1, 5, 0)]
M, N, K = 600, 520, 640


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _dev_u8(a: np.ndarray, k: int) -> torch.Tensor:
    rows = a.shape[0]
    ld = -(-k // 16) * 16
    buf = torch.zeros(rows, ld, dtype=torch.uint8, device="cuda")
    buf[:, :k] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return buf[:, :k]


def _plan(plan, cfg, slots, split):
    plan(gemm_cfg=cfg, gemm_slots=slots, gemm_split=split)


@pytest.fixture(scope="module")
def operands():
    x = bf16_host(workloads.activations(M, K, 71, 0.001))
    w = bf16_host(workloads.weights(N, K, 72))
    qa, sa = oq.quant_group(x)
    qw, sw = oq.quant_weight_block(w)
    bias = obf16.to_f64(obf16.round_from_f64(np.linspace(-2.0, 2.0, N)))
    return dict(x=x, w=w, qa=qa, sa=sa, qw=qw, sw=sw, bias=bias)


def _out():
    return padded(M, N, torch.bfloat16, 8, CANARY_BF16)


@pytest.mark.parametrize("cfg,slots,split", PLANS)
@pytest.mark.parametrize("a_layout", [0, 1])
def test_tiles_blockscale(plan, operands, cfg, slots, split, a_layout):
    log(f"tiles block cfg={cfg} slots={slots} split={split} layout={a_layout}")
    _plan(plan, cfg, slots, split)
    m = fq()
    o = operands
    sa = o["sa"].T if a_layout else o["sa"]
    yb, y = _out()
    b_d = torch.from_numpy(o["bias"].astype(np.float32)).to(torch.bfloat16).cuda()
    m.fp8q_gemm_blockscale(_dev_u8(o["qa"], K), torch.from_numpy(np.ascontiguousarray(sa)).cuda(), a_layout,
                           _dev_u8(o["qw"], K), torch.from_numpy(o["sw"]).cuda(), b_d, y, m.GRAN_BLOCK128)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_blockscale(o["qa"], o["sa"], o["qw"], o["sw"], bias=o["bias"])
    check_gemm_rows(bf16_bits(y), yr, f"block cfg={cfg} split={split}", REL)


@pytest.mark.parametrize("cfg,slots,split", PLANS)
def test_tiles_pertensor(plan, operands, cfg, slots, split):
    log(f"tiles per-tensor cfg={cfg} slots={slots} split={split}")
    _plan(plan, cfg, slots, split)
    m = fq()
    o = operands
    sx = np.float32(np.float32(np.abs(o["x"]).max()) / np.float32(448.0))
    qa = oq.quant_static(o["x"], sx)
    qw, sw = oq.quant_tensor(o["w"])
    yb, y = _out()
    m.fp8q_gemm_blockscale(_dev_u8(qa, K), torch.tensor([sx], device="cuda"), 0, _dev_u8(qw, K),
                           torch.tensor([sw], dtype=torch.float32, device="cuda"), None, y, m.GRAN_PER_TENSOR)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_pertensor(qa, sx, qw, sw)
    check_gemm_rows(bf16_bits(y), yr, f"per-tensor cfg={cfg} split={split}", REL)


@pytest.mark.parametrize("cfg,slots,split", PLANS)
def test_tiles_mxfp8(plan, operands, cfg, slots, split):
    log(f"tiles mx cfg={cfg} slots={slots} split={split}")
    _plan(plan, cfg, slots, split)
    m = fq()
    o = operands
    qa, ea = oq.quant_mx(o["x"])
    qw, ew = oq.quant_mx(o["w"])
    yb, y = _out()
    b_d = torch.from_numpy(o["bias"].astype(np.float32)).to(torch.bfloat16).cuda()
    m.fp8q_gemm_mxfp8(_dev_u8(qa, K), torch.from_numpy(ea).cuda(), _dev_u8(qw, K), torch.from_numpy(ew).cuda(),
                      b_d, y)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_mx(qa, ea, qw, ew, bias=o["bias"])
    check_gemm_rows(bf16_bits(y), yr, f"mx cfg={cfg} split={split}", REL)


def test_tiles_split_matches_unsplit(plan, operands):
    # a split tile computes the same sums in the same order: identical bits
    o = operands
    m = fq()
    outs = []
    for split in (0, 1):
        _plan(plan, 0, 6, split)
        y = m.gemm_blockscale(_dev_u8(o["qa"], K), torch.from_numpy(o["sa"]).cuda(), _dev_u8(o["qw"], K),
                              torch.from_numpy(o["sw"]).cuda())
        torch.cuda.synchronize()
        outs.append(bf16_bits(y))
    np.testing.assert_array_equal(outs[0], outs[1])
