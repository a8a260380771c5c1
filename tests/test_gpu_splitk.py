"""GPU parity of the split-K GEMM entry point.  Decode shapes whose column
tiles leave CUs idle (fp32 partial sums per K segment, added in segment
order by a second kernel): all three scale granularities, ragged M and N,
against the oracle (the method's per-row bound); repeated calls give the
same bits; a workspace too small for two segments, and shapes the split does
not serve (M > 64, or K below 96 blocks), give exactly the unsplit kernels'
bits.  Prefill shapes whose last round of tiles is at most half full (the
leftover tiles as two K halves, the second continuing from the first's
accumulators): against the oracle, bit for bit equal to the unsplit entry,
every second half recorded as having continued from the partial; and, forced
from the host, the give-up path (the second half computes the whole tile)
with the same bits."""
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
# the split serves K >= 12288 (96 blocks); (5, 300, 4096) runs unsplit
SHAPES = [(1, 2048, 14336), (16, 1024, 16384), (32, 4096, 12288), (64, 2048, 14336), (33, 1000, 12800), (5, 300, 4096)]


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _dev_u8(a, K):
    ld = -(-K // 16) * 16 + 16
    buf = torch.zeros(a.shape[0], ld, dtype=torch.uint8, device="cuda")
    buf[:, :K] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return buf[:, :K]


def _operands(M, N, K, gran, seed):
    m = fq()
    x = bf16_host(workloads.activations(M, K, seed, 0.001))
    w = bf16_host(workloads.weights(N, K, seed + 1))
    if gran == m.GRAN_PER_TENSOR:
        sx = np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))
        qa = oq.quant_static(x, sx)
        qw, sw = oq.quant_tensor(w)
        sa, sw = np.array([sx], np.float32), np.array([sw], np.float32)
        ref = lambda: og.gemm_pertensor(qa, sx, qw, sw[0])[0]
    elif gran == m.GRAN_BLOCK128_POW2:
        qa, sa = oq.quant_group_pow2(x)
        qw, sw = oq.requant_weight_pow2(*oq.quant_weight_block(w))
        ref = lambda: og.gemm_blockscale(qa, sa, qw, sw)[0]
    else:
        qa, sa = oq.quant_group(x)
        qw, sw = oq.quant_weight_block(w)
        ref = lambda: og.gemm_blockscale(qa, sa, qw, sw)[0]
    return qa, sa, qw, sw, ref


def _call(qa, sa, qw, sw, gran, ws, bias=None, a_layout=0):
    """The split entry with workspace ws (None: the unsplit entry)."""
    m = fq()
    M, K = qa.shape
    N = qw.shape[0]
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    b_d = None if bias is None else torch.from_numpy(bias.astype(np.float32)).to(torch.bfloat16).cuda()
    sa_d = torch.from_numpy(np.ascontiguousarray(sa.T if a_layout else sa)).cuda()
    sw_d = torch.from_numpy(np.ascontiguousarray(sw)).cuda()
    if ws is None:
        m.fp8q_gemm_blockscale(_dev_u8(qa, K), sa_d, a_layout, _dev_u8(qw, K), sw_d, b_d, y, gran)
    else:
        m.fp8q_gemm_blockscale_splitk(_dev_u8(qa, K), sa_d, a_layout, _dev_u8(qw, K), sw_d, b_d, y, gran, ws)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    return bf16_bits(y)


# Layout of the prefill split's workspace: per leftover tile a 256 x 256
# fp32 partial, then per leftover tile three 8-byte words (two flags and the
# outcome of the second half: tag << 32 | marker).
PARTIAL_BYTES, WORDS = 256 * 256 * 4, 3
CONSUMED, GAVE_UP = 0x5AFE0003, 0x5AFE0002


def _outcomes(ws, nbytes):
    tails = nbytes // (PARTIAL_BYTES + 8 * WORDS)
    assert tails * (PARTIAL_BYTES + 8 * WORDS) == nbytes
    words = ws.view(torch.int64)[tails * PARTIAL_BYTES // 8: tails * PARTIAL_BYTES // 8 + WORDS * tails]
    w = words.cpu().numpy().view(np.uint64).reshape(tails, WORDS)[:, 2]
    return w & np.uint64(0xFFFFFFFF), w >> np.uint64(32)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("gran", [0, 1, 2])
def test_splitk_parity(M, N, K, gran):
    m = fq()
    nbytes = m.fp8q_gemm_splitk_workspace_size(M, N, K)
    log(f"splitk M={M} N={N} K={K} gran={gran} workspace={nbytes}")
    if (M, N, K) != (5, 300, 4096):
        assert nbytes > 0, "these shapes leave CUs idle without a split"
    ws = torch.full((max(nbytes, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    qa, sa, qw, sw, ref = _operands(M, N, K, gran, M + N + K + gran)
    y = _call(qa, sa, qw, sw, gran, ws)
    check_gemm_rows(y, ref(), f"splitk M={M} N={N} K={K} gran={gran}", REL)
    np.testing.assert_array_equal(_call(qa, sa, qw, sw, gran, ws), y)      # fixed reduction order


def test_splitk_small_workspace_and_other_shapes_run_unsplit():
    m = fq()
    for (M, N, K, ws_elems) in [(16, 1024, 16384, 16 * 1024), (200, 1024, 2048, 1 << 22), (32, 2048, 7168, 1 << 22),
                                (2304, 8192, 2048, 1 << 24), (2304, 8192, 4096, 1 << 10)]:
        qa, sa, qw, sw, _ = _operands(M, N, K, 0, 7)
        ws = torch.zeros(ws_elems, dtype=torch.float32, device="cuda")    # one segment at most
        y = _call(qa, sa, qw, sw, 0, ws)
        ref = bf16_bits(m.gemm_blockscale(_dev_u8(qa, K), torch.from_numpy(sa).cuda(), _dev_u8(qw, K),
                                          torch.from_numpy(sw).cuda()))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y, ref)


def test_splitk_decode_workload_full_size():
    # the decode workload's row count with a narrow, long weight (N 2048, K 28672)
    m = fq()
    M, N, K = 32, 2048, 28672
    qa, sa, qw, sw, ref = _operands(M, N, K, 0, 99)
    nbytes = m.fp8q_gemm_splitk_workspace_size(M, N, K)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    y = _call(qa, sa, qw, sw, 0, ws)
    check_gemm_rows(y, ref(), "splitk 32x2048x7168", REL)


# Prefill shapes whose last round of 256 x 256 tiles is at most half full
# (more tiles than the 256 CUs): the leftover tiles run as two K halves
# (odd block counts included) that meet in the workspace.
# (at least 32 K blocks; 37 is odd)
PREFILL = [(2304, 8192, 4096), (2304, 8192, 4736), (2560, 7168, 6144), (4096, 6144, 6144)]


@pytest.mark.parametrize("M,N,K", PREFILL)
@pytest.mark.parametrize("gran", [0, 1, 2])
def test_prefill_tail_split_parity(M, N, K, gran):
    m = fq()
    nbytes = m.fp8q_gemm_splitk_workspace_size(M, N, K)
    log(f"prefill tail split M={M} N={N} K={K} gran={gran} workspace={nbytes}")
    assert nbytes > 0
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    qa, sa, qw, sw, ref = _operands(M, N, K, gran, M + N + K + 3 * gran)
    # a bias (added once, by the workgroup that writes the tile) and the
    # bench's column-major activation scales for the block granularities
    bias = obf16.to_f64(obf16.round_from_f64(np.linspace(-3.0, 3.0, N)))
    layout = 0 if gran == 1 else 1
    y = _call(qa, sa, qw, sw, gran, ws, bias, layout)
    rows = np.unique(np.r_[0, M - 1, np.arange(M - 256, M, 37), np.random.default_rng(5).integers(0, M, 12)])
    if gran == 1:
        yr = og.gemm_pertensor(qa, sa[0], qw, sw[0], bias=bias, rows=rows)[0]
    else:
        yr = og.gemm_blockscale(qa, sa, qw, sw, bias=bias, rows=rows)[0]
    check_gemm_rows(y[rows], yr, f"prefill split M={M} N={N} K={K}", REL)
    # every second half continued from its partner's partial, all with this
    # launch's tag
    marker, tag = _outcomes(ws, nbytes)
    assert np.all(marker == CONSUMED) and np.all(tag == tag[0]) and tag[0] != 0
    # the split keeps each element's sequence of operations: the unsplit
    # kernel's bits exactly
    np.testing.assert_array_equal(_call(qa, sa, qw, sw, gran, None, bias, layout), y)
    # fixed order, and the flags of the previous launch do not confuse the next
    np.testing.assert_array_equal(_call(qa, sa, qw, sw, gran, ws, bias, layout), y)
    marker2, tag2 = _outcomes(ws, nbytes)
    assert np.all(marker2 == CONSUMED) and np.all(tag2 != tag[0])


@pytest.mark.parametrize("gran", [0, 1, 2])
def test_prefill_tail_give_up_computes_whole_tile(plan, gran):
    """Forced from the host: every first K half publishes its partial only
    after a bounded sleep (~340 us) and every second half does not wait, so
    the second halves compute their whole tiles themselves.  The outcome
    words say so, the output keeps its bits (the same sequence of operations
    either way), and the exchange words end at their idle state: a normal
    launch afterwards continues from the partials again."""
    m = fq()
    M, N, K = 2304, 8192, 4096                       # 288 tiles: 32 leftover tiles as 64 K halves
    nbytes = m.fp8q_gemm_splitk_workspace_size(M, N, K)
    log(f"prefill tail give-up M={M} N={N} K={K} gran={gran} workspace={nbytes}")
    assert nbytes > 0
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    qa, sa, qw, sw, ref = _operands(M, N, K, gran, 7 + gran)
    layout = 0 if gran == 1 else 1
    y_split = _call(qa, sa, qw, sw, gran, ws, None, layout)
    assert np.all(_outcomes(ws, nbytes)[0] == CONSUMED)
    plan(split_wait_limit=0, split_publish_delay=100)
    y_alone = _call(qa, sa, qw, sw, gran, ws, None, layout)
    plan()
    assert np.all(_outcomes(ws, nbytes)[0] == GAVE_UP), "the give-up path was not taken"
    np.testing.assert_array_equal(y_alone, y_split)
    y_again = _call(qa, sa, qw, sw, gran, ws, None, layout)
    assert np.all(_outcomes(ws, nbytes)[0] == CONSUMED)
    np.testing.assert_array_equal(y_again, y_split)
    rows = np.unique(np.r_[2048, M - 1, np.arange(2048, M, 23), 5, 1000])
    if gran == 1:
        yr = og.gemm_pertensor(qa, sa[0], qw, sw[0], rows=rows)[0]
    else:
        yr = og.gemm_blockscale(qa, sa, qw, sw, rows=rows)[0]
    check_gemm_rows(y_alone[rows], yr, f"prefill give-up M={M} N={N} K={K}", REL)
