"""GPU parity of the grouped (MoE) block GEMM over expert-sorted rows: per
expert the block-scaled product with that expert's weight and scales, the
stacked gate/up shards of w13 with their own scale grids (shard sizes that
are and are not multiples of 128), empty experts, experts of one row and of
just more or fewer rows than a tile, both tile configurations, both
activation-scale layouts and both scale formats, against the oracle (the
method's per-row bound).  Every call goes through the C ABI."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_helpers import CANARY_BF16, bf16_bits, bf16_host, check_gemm_rows, canary_intact, log, padded

pytestmark = pytest.mark.gpu

REL = 1e-2


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _problem(counts, N, K, seed, shard=0, pow2=False):
    rng = np.random.default_rng(seed)
    M = int(sum(counts))
    x = workloads.activations(max(M, 1), K, seed, 0.001)[:M]
    xh = bf16_host(x)
    qa, sa = oq.quant_group_pow2(xh) if pow2 else oq.quant_group(xh)
    qws, sws = [], []
    for e in range(len(counts)):
        w = bf16_host(workloads.weights(N, K, seed * 100 + e))
        q, s = oq.quant_weight_block_sharded(w, shard) if shard else oq.quant_weight_block(w)
        if pow2:
            q, s = oq.requant_weight_pow2(q, s, 128, 128) if not shard else _requant_sharded(q, s, shard)
        qws.append(q)
        sws.append(s)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return qa, sa, np.stack(qws), np.stack(sws), off


def _requant_sharded(q, s, shard):
    nb = -(-shard // 128)
    parts = [oq.requant_weight_pow2(q[i:i + shard], s[(i // shard) * nb:(i // shard + 1) * nb])
             for i in range(0, q.shape[0], shard)]
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _run(qa, sa, qw, sw, off, shard, a_layout, gran):
    m = fq()
    M, K = qa.shape
    E, N, _ = qw.shape
    ld = -(-K // 16) * 16 + 16
    abuf = torch.zeros(max(M, 1), ld, dtype=torch.uint8, device="cuda")
    abuf[:M, :K] = torch.from_numpy(qa).cuda()
    a = abuf[:M, :K]
    wbuf = torch.zeros(E, N, ld, dtype=torch.uint8, device="cuda")
    wbuf[:, :, :K] = torch.from_numpy(qw).cuda()
    w = wbuf[:, :, :K]
    sa_d = torch.from_numpy(np.ascontiguousarray(sa.T if a_layout else sa)).cuda()
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_grouped_blockscale(a, sa_d, a_layout, torch.from_numpy(off).cuda(), w,
                                   torch.from_numpy(np.ascontiguousarray(sw)).cuda(), y, shard, gran)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16), "y written outside [M, N]"
    return bf16_bits(y)


CASES = [
    # (expert row counts, N, K, shard)
    ([0, 1, 37, 300, 0, 130], 384, 640, 0),
    ([255, 256, 257, 0, 513], 512, 256, 0),
    ([3, 0, 0, 64], 200, 2048, 0),
    ([129, 40, 7], 384, 512, 192),                # shard not a multiple of 128
    ([100, 300], 2 * 1088, 256, 1088),            # I_p = 1088: 2 x 9 scale rows
    ([1000, 1500, 600, 900], 1024, 1024, 512),
    # last row tiles of every height class: <= BM/2, <= 3BM/4 and above
    # (BM = 256: 150, 190, 192 and 129 take the three-quarter tile; BM = 128:
    # 90 and 96)
    ([150, 190, 193, 192, 129, 90, 96, 97], 512, 768, 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("cfg", [0, 1])
@pytest.mark.parametrize("a_layout", [0, 1])
def test_grouped_blockscale_parity(plan, case, cfg, a_layout):
    counts, N, K, shard = CASES[case]
    log(f"grouped block counts={counts} N={N} K={K} shard={shard} cfg={cfg} layout={a_layout}")
    plan(gemm_cfg=cfg)
    qa, sa, qw, sw, off = _problem(counts, N, K, 11 + case, shard)
    y = _run(qa, sa, qw, sw, off, shard, a_layout, fq().GRAN_BLOCK128)
    yr = og.gemm_grouped_blockscale(qa, sa, qw, sw, off, shard=shard)
    check_gemm_rows(y, yr, f"grouped case {case}", REL)


@pytest.mark.parametrize("case", [0, 3, 5])
@pytest.mark.parametrize("cfg", [0, 1])
def test_grouped_pow2_parity(plan, case, cfg):
    counts, N, K, shard = CASES[case]
    log(f"grouped pow2 counts={counts} N={N} K={K} shard={shard} cfg={cfg}")
    plan(gemm_cfg=cfg)
    qa, sa, qw, sw, off = _problem(counts, N, K, 31 + case, shard, pow2=True)
    y = _run(qa, sa, qw, sw, off, shard, 1, fq().GRAN_BLOCK128_POW2)
    yr = og.gemm_grouped_blockscale(qa, sa, qw, sw, off, shard=shard)
    check_gemm_rows(y, yr, f"grouped pow2 case {case}", REL)


def test_grouped_equals_dense_per_expert():
    # each expert's rows through the grouped kernel and through the dense
    # fast kernel: the same tile code, so the same bits
    m = fq()
    counts, N, K = [300, 0, 520, 77], 768, 1024
    qa, sa, qw, sw, off = _problem(counts, N, K, 41)
    y = _run(qa, sa, qw, sw, off, 0, 0, m.GRAN_BLOCK128)
    for e in range(len(counts)):
        r = slice(off[e], off[e + 1])
        if off[e + 1] - off[e] <= 64:
            continue                                  # dense path takes its decode kernel there
        ld = -(-K // 16) * 16
        a = torch.zeros(off[e + 1] - off[e], ld, dtype=torch.uint8, device="cuda")
        a[:, :K] = torch.from_numpy(qa[r]).cuda()
        wd = torch.zeros(N, ld, dtype=torch.uint8, device="cuda")
        wd[:, :K] = torch.from_numpy(qw[e]).cuda()
        yd = m.gemm_blockscale(a[:, :K], torch.from_numpy(np.ascontiguousarray(sa[r])).cuda(), wd[:, :K],
                               torch.from_numpy(sw[e]).cuda())
        torch.cuda.synchronize()
        yr = og.gemm_blockscale(qa[r], sa[r], qw[e], sw[e])[0]
        check_gemm_rows(bf16_bits(yd), yr, f"dense expert {e}", REL)
        check_gemm_rows(y[r], yr, f"grouped expert {e}", REL)


def test_grouped_deterministic():
    m = fq()
    qa, sa, qw, sw, off = _problem([400, 10, 900], 512, 1024, 51)
    y1 = _run(qa, sa, qw, sw, off, 0, 1, m.GRAN_BLOCK128)
    y2 = _run(qa, sa, qw, sw, off, 0, 1, m.GRAN_BLOCK128)
    np.testing.assert_array_equal(y1, y2)


@pytest.mark.parametrize("name", ["moe_up", "moe_down"])
def test_grouped_full_size_sampled_rows(name):
    # the bench's launch configuration (GPU quantizers, column-major
    # activation scales) on the MoE layer share, oracle on sampled rows of
    # three experts
    m = fq()
    wl = workloads.MOE_WORKLOADS[name]
    _, off = wl.routing()
    M, N, K, E = int(off[-1]), wl.N, wl.K, wl.local_experts
    log(f"grouped full size {name}: M={M} N={N} K={K} E={E} shard={wl.shard}")
    x = wl.activations()
    qa, sa = m.quant_act_group(x.cuda(), layout=m.COL_MAJOR)
    qw = torch.empty(E, N, K, dtype=torch.uint8, device="cuda")
    nbs = (N // wl.shard) * math.ceil(wl.shard / 128) if wl.shard else math.ceil(N / 128)
    sw = torch.empty(E, nbs, K // 128, dtype=torch.float32, device="cuda")
    for e in range(E):
        wd = wl.expert_weight(e).cuda()
        if wl.shard:
            nb = math.ceil(wl.shard / 128)
            for i in range(N // wl.shard):
                m.fp8q_quant_weight_block(wd[i * wl.shard:(i + 1) * wl.shard], 128, 128, m.SCALE_F32,
                                          qw[e, i * wl.shard:(i + 1) * wl.shard], sw[e, i * nb:(i + 1) * nb])
        else:
            m.fp8q_quant_weight_block(wd, 128, 128, m.SCALE_F32, qw[e], sw[e])
    y = m.gemm_grouped_blockscale(qa, sa, off.to(torch.int32).cuda(), qw, sw, shard=wl.shard, a_layout=m.COL_MAJOR)
    torch.cuda.synchronize()
    experts = [0, E // 2, E - 1]
    rows = np.concatenate([[off[e].item(), off[e].item() + 1, off[e + 1].item() - 1] for e in experts])
    xh = bf16_host(x[rows])
    qa_r, sa_r = oq.quant_group(xh)
    cache = {}

    def w_of(e):
        if e not in cache:
            wh = bf16_host(wl.expert_weight(int(e)))
            cache[e] = oq.quant_weight_block_sharded(wh, wl.shard) if wl.shard else oq.quant_weight_block(wh)
        return cache[e]

    off_np = off.numpy()
    yr = np.empty((len(rows), N), np.uint16)
    for i, r in enumerate(rows):
        e = int(np.searchsorted(off_np, r, side="right") - 1)
        q, s = w_of(e)
        yr[i] = og.gemm_blockscale(qa_r[i:i + 1], sa_r[i:i + 1], q, s, shard=wl.shard)[0][0]
    check_gemm_rows(bf16_bits(y)[rows], yr, f"full {name}", REL)
