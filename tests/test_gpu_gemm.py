"""GPU parity of the scaled GEMMs against the CPU oracle.

Quantized operands are produced by the ORACLE quantizers on the CPU and
uploaded, so the GEMM is checked on inputs that owe nothing to the HIP path.
Tolerance (stated by the method): per output row,
max |Y_gpu - Y_oracle| <= 1e-2 * max |Y_oracle| after bf16 rounding.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import bf16 as obf16
from oracle import e4m3, gemm as og
from oracle import quant as oq
from tests.gpu_helpers import CANARY_BF16, bf16_bits, bf16_host, canary_intact, check_gemm_rows, log, padded

pytestmark = pytest.mark.gpu

REL = 1e-2


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _dev_u8(a: np.ndarray, K: int) -> torch.Tensor:
    """uint8 [rows, K] numpy -> device view with a 16-byte-aligned row stride."""
    rows = a.shape[0]
    ld = -(-K // 16) * 16
    buf = torch.zeros(rows, ld, dtype=torch.uint8, device="cuda")
    buf[:, :K] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return buf[:, :K]


def _problem(M, N, K, seed, outliers=0.001, w_std=None):
    x = workloads.activations(M, K, seed, outliers)
    w = workloads.weights(N, K, seed + 1, w_std)
    qa, sa = oq.quant_group(bf16_host(x))
    qw, sw = oq.quant_weight_block(bf16_host(w))
    return x, w, qa, sa, qw, sw


def _run_block(qa, sa, qw, sw, bias=None, a_layout=0):
    m = fq()
    M, K = qa.shape
    N = qw.shape[0]
    a = _dev_u8(qa, K)
    wd = _dev_u8(qw, K)
    sa_d = torch.from_numpy(np.ascontiguousarray(sa.T if a_layout else sa)).cuda()
    sw_d = torch.from_numpy(sw).cuda()
    b_d = None
    if bias is not None:
        b_d = torch.from_numpy(bias.astype(np.float32)).to(torch.bfloat16).cuda()
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_blockscale(a, sa_d, a_layout, wd, sw_d, b_d, y, m.GRAN_BLOCK128)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16), "y written outside [M, N]"
    return bf16_bits(y)


# prefill path (M > 64) and decode path (M <= 64), ragged M / N / K
SHAPES = [
    (16, 256, 512), (5, 300, 520), (33, 130, 128), (64, 576, 6144), (1, 96, 200),
    (65, 576, 6144), (130, 2048, 1000), (200, 256, 7168), (256, 384, 640), (17, 1536, 6144),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_blockscale_parity(M, N, K):
    log(f"gemm_blockscale M={M} N={N} K={K}")
    _, _, qa, sa, qw, sw = _problem(M, N, K, seed=M + N + K)
    y = _run_block(qa, sa, qw, sw)
    yr, _ = og.gemm_blockscale(qa, sa, qw, sw)
    check_gemm_rows(y, yr, f"block M={M} N={N} K={K}", REL)


@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (100, 300, 520)])
def test_gemm_blockscale_bias_and_col_major_scales(M, N, K):
    log(f"gemm_blockscale bias/col-major M={M} N={N} K={K}")
    _, _, qa, sa, qw, sw = _problem(M, N, K, seed=3 * M + K)
    bias = obf16.to_f64(obf16.round_from_f64(np.linspace(-1.5, 1.5, N)))
    y = _run_block(qa, sa, qw, sw, bias=bias, a_layout=1)
    yr, _ = og.gemm_blockscale(qa, sa, qw, sw, bias=bias)
    check_gemm_rows(y, yr, "block bias col-major", REL)


@pytest.mark.parametrize("M", [254, 40])
def test_gemm_exhaustive_code_products(M):
    # one non-zero per row, unit scales: Y[i,j] = dec(a_i) * dec(w_j), exact in
    # bf16 -> the kernel must reproduce every product exactly
    log(f"gemm exhaustive code products (M={M})")
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    qa = np.zeros((M, 128), np.uint8)
    qa[:, 0] = codes[:M]
    qw = np.zeros((codes.size, 128), np.uint8)
    qw[:, 0] = codes
    sa = np.ones((M, 1), np.float32)
    sw = np.ones((2, 1), np.float32)
    y = _run_block(qa, sa, qw, sw)
    yr, _ = og.gemm_blockscale(qa, sa, qw, sw)
    np.testing.assert_array_equal(obf16.to_f64(y), obf16.to_f64(yr))


@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (5, 300, 520), (130, 640, 2048), (48, 1536, 7168)])
def test_gemm_pertensor_parity(M, N, K):
    log(f"gemm_pertensor M={M} N={N} K={K}")
    m = fq()
    x = workloads.activations(M, K, seed=K + 1)
    w = workloads.weights(N, K, seed=K + 2, std=1.0)
    xh = bf16_host(x)
    sx = np.float32(np.float32(np.abs(xh).max()) / np.float32(448.0))
    qa = oq.quant_static(xh, sx)
    qw, sw = oq.quant_tensor(bf16_host(w))
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_blockscale(_dev_u8(qa, K), torch.tensor([sx], device="cuda"), 0, _dev_u8(qw, K),
                           torch.tensor([sw], dtype=torch.float32, device="cuda"), None, y,
                           m.GRAN_PER_TENSOR)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_pertensor(qa, sx, qw, sw)
    check_gemm_rows(bf16_bits(y), yr, f"per-tensor M={M} N={N} K={K}", REL)


@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (5, 300, 520), (100, 640, 7168), (64, 256, 200)])
def test_gemm_mxfp8_parity(M, N, K):
    log(f"gemm_mxfp8 M={M} N={N} K={K}")
    m = fq()
    x = workloads.activations(M, K, seed=K + 7)
    w = workloads.weights(N, K, seed=K + 8, std=1.0)
    qa, ea = oq.quant_mx(bf16_host(x))
    qw, ew = oq.quant_mx(bf16_host(w))
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_mxfp8(_dev_u8(qa, K), torch.from_numpy(ea).cuda(), _dev_u8(qw, K),
                      torch.from_numpy(ew).cuda(), None, y)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_mx(qa, ea, qw, ew)
    check_gemm_rows(bf16_bits(y), yr, f"mx M={M} N={N} K={K}", REL)


# column-major MX scales ([K/32, rows]): the fast kernel in both tile
# configurations (and its half-height tail), ragged N and M (multiples of 4)
@pytest.mark.parametrize("M,N,K", [(100, 640, 7168), (260, 1028, 1024), (2048, 7168, 1024), (516, 2052, 2048),
                                   (1540, 4096, 512)])
@pytest.mark.parametrize("cfg", [0, 1])
def test_gemm_mxfp8_col_major_scales(plan, M, N, K, cfg):
    log(f"gemm_mxfp8 col-major M={M} N={N} K={K} cfg={cfg}")
    plan(gemm_cfg=cfg)
    m = fq()
    x = workloads.activations(M, K, seed=K + 17, outlier_frac=0.001)
    w = workloads.weights(N, K, seed=K + 18, std=1.0)
    qa, ea = oq.quant_mx(bf16_host(x))
    qw, ew = oq.quant_mx(bf16_host(w))
    bias = obf16.to_f64(obf16.round_from_f64(np.linspace(-2.0, 2.0, N)))
    b_d = torch.from_numpy(bias.astype(np.float32)).to(torch.bfloat16).cuda()
    yb, y = padded(M, N, torch.bfloat16, 8, CANARY_BF16)
    m.fp8q_gemm_mxfp8(_dev_u8(qa, K), torch.from_numpy(np.ascontiguousarray(ea.T)).cuda(), _dev_u8(qw, K),
                      torch.from_numpy(np.ascontiguousarray(ew.T)).cuda(), b_d, y, m.COL_MAJOR)
    torch.cuda.synchronize()
    assert canary_intact(yb, N, CANARY_BF16)
    yr, _ = og.gemm_mx(qa, ea, qw, ew, bias=bias)
    check_gemm_rows(bf16_bits(y), yr, f"mx col-major M={M} N={N} K={K}", REL)


def test_gemm_mx_scale_placement():
    # distinct power-of-two scale per 32-block: any mix-up of which block a
    # scale byte applies to changes the result far beyond the tolerance
    log("gemm_mxfp8 scale placement")
    m = fq()
    M, N, K = 32, 64, 256
    rng = np.random.default_rng(5)
    qa = rng.choice(np.array([0x38, 0xB8, 0x40, 0x30], np.uint8), size=(M, K))   # +-1, 2, 0.5
    qw = rng.choice(np.array([0x38, 0xB8, 0x44], np.uint8), size=(N, K))
    ea = (127 + rng.integers(-6, 7, size=(M, K // 32))).astype(np.uint8)
    ew = (127 + rng.integers(-6, 7, size=(N, K // 32))).astype(np.uint8)
    y = m.gemm_mxfp8(_dev_u8(qa, K), torch.from_numpy(ea).cuda(), _dev_u8(qw, K), torch.from_numpy(ew).cuda())
    torch.cuda.synchronize()
    yr, _ = og.gemm_mx(qa, ea, qw, ew)
    check_gemm_rows(bf16_bits(y), yr, "mx placement", REL)


def test_gemm_deterministic():
    log("gemm determinism")
    _, _, qa, sa, qw, sw = _problem(300, 512, 2048, seed=42)
    y1 = _run_block(qa, sa, qw, sw)
    y2 = _run_block(qa, sa, qw, sw)
    np.testing.assert_array_equal(y1, y2)
    _, _, qa, sa, qw, sw = _problem(32, 1536, 2048, seed=43)
    np.testing.assert_array_equal(_run_block(qa, sa, qw, sw), _run_block(qa, sa, qw, sw))


def _full_size(name, rows_sample):
    """Full-size workload: GPU quantizes and multiplies (as the bench does);
    the oracle recomputes sampled output rows from the same bf16 inputs."""
    m = fq()
    wl = workloads.WORKLOADS[name]
    d = wl.make("cpu")
    log(f"full size {name}: M={wl.M} N={wl.N} K={wl.K}")
    xd, wd = d["x"].cuda(), d["w"].cuda()
    qw, sw = m.quant_weight_block(wd)
    # the bench's launch configuration: column-major activation scales
    if wl.norm:
        qa, sa = m.rmsnorm_quant(xd, d["gamma"].cuda(), d["eps"], layout=m.COL_MAJOR)
    else:
        qa, sa = m.quant_act_group(xd, layout=m.COL_MAJOR)
    y = m.gemm_blockscale(qa, sa, qw, sw, a_layout=m.COL_MAJOR)
    # and the bench's own call: the split-K entry with the workspace the
    # library asks for (the prefill shape splits its leftover tiles along K)
    y_split = m.gemm_blockscale_splitk(qa, sa, qw, sw, a_layout=m.COL_MAJOR)
    torch.cuda.synchronize()
    rows = rows_sample(wl.M)
    xh = bf16_host(d["x"][rows])
    if wl.norm:
        ref = oq.rmsnorm_quant(xh, bf16_host(d["gamma"]), d["eps"])
        qa_r, sa_r = ref["q"], ref["s"]
    else:
        qa_r, sa_r = oq.quant_group(xh)
    qw_r, sw_r = oq.quant_weight_block(bf16_host(d["w"]))
    yr, _ = og.gemm_blockscale(qa_r, sa_r, qw_r, sw_r)
    check_gemm_rows(bf16_bits(y)[rows], yr, f"full {name}", REL)
    check_gemm_rows(bf16_bits(y_split)[rows], yr, f"full {name} (split-K entry)", REL)


def test_full_size_decode():
    _full_size("decode", lambda M: np.arange(M))


def test_full_size_prefill_norm():
    # sampled rows include the last 256 (the split tail tiles' rows)
    _full_size("prefill_norm", lambda M: np.unique(np.r_[0, M - 1, np.arange(M - 256, M, 31),
                                                       np.random.default_rng(2).integers(0, M, 14)]))


def test_full_size_large():
    _full_size("large", lambda M: np.unique(np.r_[0, M - 1, np.random.default_rng(3).integers(0, M, 6)]))


def test_full_size_mx_and_pertensor():
    m = fq()
    wl = workloads.WORKLOADS["mx"]
    d = wl.make("cpu")
    log(f"full size mx: M={wl.M} N={wl.N} K={wl.K}")
    xd, wd = d["x"].cuda(), d["w"].cuda()
    qa, ea = m.quant_act_mx(xd)
    qw, ew = m.quant_weight_mx(wd)
    y = m.gemm_mxfp8(qa, ea, qw, ew)
    # the bench's configuration: column-major scales from the same quantizer
    qa_c, ea_c = m.quant_act_mx(xd, layout=m.COL_MAJOR)
    qw_c, ew_c = m.quant_act_mx(wd, layout=m.COL_MAJOR)
    y_c = m.gemm_mxfp8(qa_c, ea_c, qw_c, ew_c, scale_layout=m.COL_MAJOR)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ea_c.cpu().numpy().T, ea.cpu().numpy())
    np.testing.assert_array_equal(ew_c.cpu().numpy().T, ew.cpu().numpy())
    rows = np.unique(np.r_[0, wl.M - 1, np.random.default_rng(4).integers(0, wl.M, 6)])
    qa_r, ea_r = oq.quant_mx(bf16_host(d["x"][rows]))
    qw_r, ew_r = oq.quant_mx(bf16_host(d["w"]))
    yr, _ = og.gemm_mx(qa_r, ea_r, qw_r, ew_r)
    check_gemm_rows(bf16_bits(y)[rows], yr, "full mx", REL)
    check_gemm_rows(bf16_bits(y_c)[rows], yr, "full mx col-major", REL)
    # per-tensor static on the same shapes
    xh = bf16_host(d["x"])
    sx = np.float32(np.float32(np.abs(xh).max()) / np.float32(448.0))
    qa2 = m.quant_act_static(xd, torch.tensor([sx], device="cuda"))
    qw2, sw2 = m.quant_weight_tensor(wd)
    y2 = m.gemm_pertensor(qa2, torch.tensor([sx], device="cuda"), qw2, sw2)
    torch.cuda.synchronize()
    qa2_r = oq.quant_static(xh[rows], sx)
    qw2_r, sw2_r = oq.quant_tensor(bf16_host(d["w"]))
    yr2, _ = og.gemm_pertensor(qa2_r, sx, qw2_r, sw2_r)
    check_gemm_rows(bf16_bits(y2)[rows], yr2, "full per-tensor", REL)
