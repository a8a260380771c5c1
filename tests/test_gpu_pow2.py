"""GPU parity of the power-of-two scale path (block FP8 consumed as an MXFP8
view): the group-128 activation quantizer and the fused RMSNorm front end
with power-of-two scales, the 128x128 weight quantizer, the re-quantization
of fp32-scaled blocks (codes and scales bit for bit), and the GEMM whose
scaled MFMAs apply the scales' exponent bytes (the method's per-row bound).
Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import workloads
from oracle import bf16 as obf16
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_helpers import CANARY_BF16, CANARY_U8, bf16_bits, bf16_host, canary_intact, check_gemm_rows, log, padded
from tests.test_gpu_quant import _special_rows

pytestmark = pytest.mark.gpu

REL = 1e-2


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _dev_u8(a: np.ndarray, K: int) -> torch.Tensor:
    rows = a.shape[0]
    ld = -(-K // 16) * 16 + 16
    buf = torch.zeros(rows, ld, dtype=torch.uint8, device="cuda")
    buf[:, :K] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return buf[:, :K]


@pytest.mark.parametrize("M,K", [(16, 512), (5, 520), (3, 1001), (33, 6144), (2, 8), (1, 7168), (70, 300),
                                 (7, 2560), (6, 3584)])
@pytest.mark.parametrize("layout", [0, 1])
def test_quant_group_pow2_parity(M, K, layout):
    log(f"quant_group pow2 M={M} K={K} layout={layout}")
    m = fq()
    x = workloads.activations(M, K, seed=M * 5 + K, outlier_frac=0.001)
    xb, xd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    xd.copy_(x.cuda())
    qb, q = padded(M, K, torch.uint8, 16, CANARY_U8)
    G = -(-K // 128)
    s = torch.empty((G, M) if layout else (M, G), dtype=torch.float32, device="cuda")
    m.fp8q_quant_act_group(xd, 128, m.SCALE_F32_POW2, layout, None, q, s)
    torch.cuda.synchronize()
    assert canary_intact(qb, K, CANARY_U8)
    qr, sr = oq.quant_group_pow2(bf16_host(x))
    sg = s.cpu().numpy()
    np.testing.assert_array_equal(sg.T if layout else sg, sr)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


@pytest.mark.parametrize("K", [512, 1000])
def test_quant_group_pow2_special_values(K):
    m = fq()
    x = _special_rows(K, seed=K + 3)
    q, s = m.quant_act_group_pow2(x.cuda())
    torch.cuda.synchronize()
    qr, sr = oq.quant_group_pow2(bf16_host(x))
    np.testing.assert_array_equal(s.cpu().numpy(), sr)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


@pytest.mark.parametrize("M,K", [(16, 512), (5, 520), (64, 6144), (3, 7168), (2, 1001), (2500, 6144), (3, 17000)])
@pytest.mark.parametrize("add", [False, True])
def test_norm_pow2_parity(M, K, add):
    log(f"rmsnorm pow2 M={M} K={K} add={add}")
    m = fq()
    x = workloads.activations(M, K, seed=K + 51, outlier_frac=0.001)
    h = (workloads.activations(M, K, seed=K + 52, outlier_frac=0.001).float() * 0.25).to(torch.bfloat16)
    g = workloads.gamma(K, seed=K + 53)
    _, xd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    xd.copy_(x.cuda())
    hd = None
    if add:
        _, hd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
        hd.copy_(h.cuda())
    qb, q = padded(M, K, torch.uint8, 16, CANARY_U8)
    G = -(-K // 128)
    s = torch.empty(G, M, dtype=torch.float32, device="cuda")
    m.fp8q_add_rmsnorm_quant(xd, hd, xd if add else None, g.cuda(), 1e-6, m.SCALE_F32_POW2, m.COL_MAJOR, None,
                             q, s)
    torch.cuda.synchronize()
    assert canary_intact(qb, K, CANARY_U8)
    xh, gh = bf16_host(x), bf16_host(g)
    hh = bf16_host(h) if add else np.zeros_like(xh)
    ref = oq.add_rmsnorm_quant(xh, hh, gh, 1e-6, pow2=True)
    if add:
        np.testing.assert_array_equal(bf16_bits(xd), ref["z"])
    qg, sg = q.cpu().numpy(), s.cpu().numpy().T
    amb = np.flatnonzero(ref["ambiguous"])
    ok = np.ones(M, bool)
    ok[amb] = False
    np.testing.assert_array_equal(qg[ok], ref["q"][ok])
    np.testing.assert_array_equal(sg[ok], ref["s"][ok])
    for i in amb:
        r_alt = ref["r"].copy()
        r_alt[i] = ref["r_alt"][i]
        alt = oq.add_rmsnorm_quant(xh, hh, gh, 1e-6, pow2=True, r=r_alt)
        assert any(np.array_equal(qg[i], c["q"][i]) and np.array_equal(sg[i], c["s"][i]) for c in (ref, alt))


@pytest.mark.parametrize("N,K", [(256, 512), (300, 200), (128, 1001), (1024, 7168)])
def test_weight_block_pow2_parity(N, K):
    log(f"weight pow2 N={N} K={K}")
    m = fq()
    w = workloads.weights(N, K, seed=N + K + 61)
    _, wd = padded(N, K, torch.bfloat16, 8, CANARY_BF16)
    wd.copy_(w.cuda())
    q, s = m.quant_weight_block_pow2(wd)
    torch.cuda.synchronize()
    qr, sr = oq.quant_weight_block_pow2(bf16_host(w))
    np.testing.assert_array_equal(s.cpu().numpy(), sr)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


@pytest.mark.parametrize("N,K", [(256, 512), (300, 200), (129, 1001), (1024, 7168)])
@pytest.mark.parametrize("inplace", [False, True])
def test_requant_pow2_parity(N, K, inplace):
    log(f"requant pow2 N={N} K={K} inplace={inplace}")
    m = fq()
    w = workloads.weights(N, K, seed=N + K + 71)
    qw, sw = oq.quant_weight_block(bf16_host(w))           # an fp32-scaled block-FP8 checkpoint
    q_in = _dev_u8(qw, K)
    s_in = torch.from_numpy(sw).cuda()
    if inplace:
        q_out, s_out = q_in, s_in
    else:
        qb, q_out = padded(N, K, torch.uint8, 16, CANARY_U8)
        s_out = torch.empty_like(s_in)
    m.fp8q_requant_weight_pow2(q_in, s_in, q_out, s_out)
    torch.cuda.synchronize()
    if not inplace:
        assert canary_intact(qb, K, CANARY_U8)
        np.testing.assert_array_equal(q_in.cpu().numpy(), qw)              # input untouched
    qr, sr = oq.requant_weight_pow2(qw, sw)
    np.testing.assert_array_equal(s_out.cpu().numpy(), sr)
    np.testing.assert_array_equal(q_out.cpu().numpy(), qr)


def _pow2_problem(M, N, K, seed):
    x = workloads.activations(M, K, seed, 0.001)
    w = workloads.weights(N, K, seed + 1)
    qa, sa = oq.quant_group_pow2(bf16_host(x))
    qw, sw = oq.requant_weight_pow2(*oq.quant_weight_block(bf16_host(w)))
    return qa, sa, qw, sw


# fast kernel (M > 64, K % 128 == 0) in both tile configurations and the
# half-height tail, plus the shapes the block-mode kernels take
SHAPES = [(65, 576, 6144), (256, 384, 640), (300, 1000, 1024), (1024, 2048, 2048), (2048, 7168, 1024),
          (130, 2048, 1000), (16, 256, 512), (64, 576, 6144), (5, 300, 520)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("a_layout", [0, 1])
def test_gemm_pow2_parity(M, N, K, a_layout):
    log(f"gemm pow2 M={M} N={N} K={K} layout={a_layout}")
    m = fq()
    qa, sa, qw, sw = _pow2_problem(M, N, K, seed=M + N + K + 81)
    bias = obf16.to_f64(obf16.round_from_f64(np.linspace(-2.0, 2.0, N)))
    b_d = torch.from_numpy(bias.astype(np.float32)).to(torch.bfloat16).cuda()
    sa_d = torch.from_numpy(np.ascontiguousarray(sa.T if a_layout else sa)).cuda()
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_blockscale(_dev_u8(qa, K), sa_d, a_layout, _dev_u8(qw, K), torch.from_numpy(sw).cuda(), b_d, y,
                           m.GRAN_BLOCK128_POW2)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_blockscale(qa, sa, qw, sw, bias=bias)
    check_gemm_rows(bf16_bits(y), yr, f"pow2 M={M} N={N} K={K}", REL)


def test_gemm_pow2_matches_block_mode_closely():
    # the same power-of-two scales through the VALU-rescale kernel: the two
    # sums differ only in rounding order
    m = fq()
    M, N, K = 512, 1024, 4096
    qa, sa, qw, sw = _pow2_problem(M, N, K, seed=91)
    args = (_dev_u8(qa, K), torch.from_numpy(sa).cuda(), _dev_u8(qw, K), torch.from_numpy(sw).cuda())
    y1 = obf16.to_f64(bf16_bits(m.gemm_blockscale_pow2(*args)))
    y2 = obf16.to_f64(bf16_bits(m.gemm_blockscale(*args)))
    torch.cuda.synchronize()
    scale = np.max(np.abs(y2), axis=1, keepdims=True)
    assert np.max(np.abs(y1 - y2) / scale) <= 2.0 ** -7


def test_gemm_pow2_deterministic():
    m = fq()
    qa, sa, qw, sw = _pow2_problem(512, 1536, 2048, seed=93)
    args = (_dev_u8(qa, 2048), torch.from_numpy(sa).cuda(), _dev_u8(qw, 2048), torch.from_numpy(sw).cuda())
    np.testing.assert_array_equal(bf16_bits(m.gemm_blockscale_pow2(*args)), bf16_bits(m.gemm_blockscale_pow2(*args)))


def test_full_size_large_pow2():
    # the bench's launch configuration: GPU quantizers (pow2 activations,
    # requantized block weights), column-major activation scales
    m = fq()
    wl = workloads.WORKLOADS["large"]
    d = wl.make("cpu")
    log(f"full size large pow2: M={wl.M} N={wl.N} K={wl.K}")
    qw0, sw0 = m.quant_weight_block(d["w"].cuda())
    qw, sw = m.requant_weight_pow2(qw0, sw0)
    qa, sa = m.quant_act_group_pow2(d["x"].cuda(), layout=m.COL_MAJOR)
    y = m.gemm_blockscale_pow2(qa, sa, qw, sw, a_layout=m.COL_MAJOR)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, wl.M - 1, np.random.default_rng(4).integers(0, wl.M, 6)])
    qa_r, sa_r = oq.quant_group_pow2(bf16_host(d["x"][rows]))
    qw_r, sw_r = oq.requant_weight_pow2(*oq.quant_weight_block(bf16_host(d["w"])))
    np.testing.assert_array_equal(sw.cpu().numpy(), sw_r)
    yr, _ = og.gemm_blockscale(qa_r, sa_r, qw_r, sw_r)
    check_gemm_rows(bf16_bits(y)[rows], yr, "full large pow2", REL)
