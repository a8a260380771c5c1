"""GPU parity of the quantizers against the CPU oracle: bit-exact codes and
scales.  Every call goes through the C ABI (fp8_block_scaled_token_amd)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import bf16 as obf16
from oracle import quant as oq
from tests.gpu_helpers import CANARY_BF16, CANARY_U8, bf16_bits, bf16_host, canary_intact, log, padded

pytestmark = pytest.mark.gpu


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _special_rows(K, seed):
    """bf16 rows with the degenerate cases: zero row, -0, tiny and subnormal
    values, huge values, exact E4M3 values, a single non-zero per group."""
    rng = np.random.default_rng(seed)
    rows = np.zeros((8, K), np.float32)
    rows[1] = -0.0
    rows[2] = rng.standard_normal(K) * 1e-39          # bf16 subnormals
    rows[3] = rng.standard_normal(K) * 1e30
    rows[4] = rng.standard_normal(K) * 1e-12          # below the 1e-10 floor
    rows[5, ::128] = 3.0                              # one value per group
    rows[6] = rng.choice([-448.0, -1.5, 0.0, 2.0 ** -9, 448.0, 3.25], K)
    rows[7] = rng.standard_normal(K)
    rows[7, 5] = -3.0e38
    return torch.from_numpy(rows).to(torch.bfloat16)


def _run_group128(x_cpu, layout):
    m = fq()
    M, K = x_cpu.shape
    xb, x = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    x.copy_(x_cpu.cuda())
    qb, q = padded(M, K, torch.uint8, 16, CANARY_U8)
    G = -(-K // 128)
    s = torch.empty((G, M) if layout == m.COL_MAJOR else (M, G), dtype=torch.float32, device="cuda")
    m.fp8q_quant_act_group(x, 128, m.SCALE_F32, layout, None, q, s)
    torch.cuda.synchronize()
    assert canary_intact(qb, K, CANARY_U8), "q written outside [M, K]"
    s = s.cpu().numpy()
    if layout == m.COL_MAJOR:
        s = s.T
    return q.cpu().numpy(), s


@pytest.mark.parametrize("M,K", [(16, 512), (5, 520), (3, 1001), (33, 6144), (2, 8), (1, 7168), (70, 300),
                                 (9, 1536), (7, 2560), (6, 3584)])   # 3, 5, 7 chunks per wave
@pytest.mark.parametrize("layout", [0, 1])
def test_quant_group128_parity(M, K, layout):
    log(f"quant_group128 M={M} K={K} layout={layout}")
    x = workloads.activations(M, K, seed=M * 7 + K, outlier_frac=0.001)
    q, s = _run_group128(x, layout)
    qr, sr = oq.quant_group(bf16_host(x))
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(q, qr)


@pytest.mark.parametrize("K", [384, 520])
def test_quant_group128_special_values(K):
    log(f"quant_group128 special K={K}")
    x = _special_rows(K, K)
    q, s = _run_group128(x, 0)
    qr, sr = oq.quant_group(bf16_host(x))
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(q, qr)


@pytest.mark.parametrize("name", ["large", "decode"])
def test_quant_group128_full_size_sampled_rows(name):
    wl = workloads.WORKLOADS[name]
    log(f"quant_group128 full size {name} [{wl.M},{wl.K}]")
    m = fq()
    x = workloads.activations(wl.M, wl.K, wl.seed * 10 + 1, wl.outlier_frac, device="cpu")
    q, s = m.quant_act_group(x.cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, wl.M - 1], np.random.default_rng(0).integers(0, wl.M, 30)]))
    qr, sr = oq.quant_group(bf16_host(x[rows]))
    np.testing.assert_array_equal(s.cpu().numpy()[rows], sr)
    np.testing.assert_array_equal(q.cpu().numpy()[rows], qr)


@pytest.mark.parametrize("M,K", [(16, 512), (5, 200), (3, 1001), (9, 7168), (9, 1536), (7, 2560), (6, 3584)])
def test_quant_mx_parity(M, K):
    log(f"quant_mx M={M} K={K}")
    m = fq()
    x = workloads.activations(M, K, seed=K + 3, outlier_frac=0.001)
    xb, xd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    xd.copy_(x.cuda())
    qb, q = padded(M, K, torch.uint8, 16, CANARY_U8)
    s = torch.empty(M, -(-K // 32), dtype=torch.uint8, device="cuda")
    m.fp8q_quant_act_group(xd, 32, m.SCALE_UE8M0, m.ROW_MAJOR, None, q, s)
    torch.cuda.synchronize()
    assert canary_intact(qb, K, CANARY_U8)
    qr, sr = oq.quant_mx(bf16_host(x))
    np.testing.assert_array_equal(s.cpu().numpy(), sr)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


def test_quant_mx_special_values():
    log("quant_mx special")
    m = fq()
    x = _special_rows(256, 1)
    q, s = m.quant_act_mx(x.cuda())
    torch.cuda.synchronize()
    qr, sr = oq.quant_mx(bf16_host(x))
    np.testing.assert_array_equal(s.cpu().numpy(), sr)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


@pytest.mark.parametrize("M,K", [(16, 512), (5, 520), (64, 7168), (9, 1536), (7, 2560), (6, 3584), (3, 9000)])
def test_quant_static_parity(M, K):
    log(f"quant_static M={M} K={K}")
    m = fq()
    x = workloads.activations(M, K, seed=K + 5, outlier_frac=0.001)
    xh = bf16_host(x)
    # calibration stand-in: max |A| / 448 over this batch, in fp32
    sx = np.float32(np.float32(np.abs(xh).max()) / np.float32(448.0))
    sd = torch.tensor([sx], dtype=torch.float32, device="cuda")
    q = m.quant_act_static(x.cuda(), sd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), oq.quant_static(xh, sx))
    # a scale that saturates part of the row
    sd2 = torch.tensor([sx / 4], dtype=torch.float32, device="cuda")
    q2 = m.quant_act_static(x.cuda(), sd2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q2.cpu().numpy(), oq.quant_static(xh, np.float32(sx / 4)))


def _rms_expected(xh, gh, eps, y_gpu_bits):
    """Oracle result; near-tie rows accept either neighbouring fp32 r."""
    ref = oq.rmsnorm_quant(xh, gh, eps)
    amb = np.flatnonzero(ref["ambiguous"])
    if amb.size:
        log(f"  near-tie rows: {amb.tolist()}")
    return ref, amb


# several rows per workgroup with a short last run (2500 rows at K 6144 and
# 1030 rows at K 16384), and rows longer than the one-read limit (17000)
@pytest.mark.parametrize("M,K", [(16, 512), (5, 520), (64, 6144), (3, 7168), (4, 9000), (2, 1001),
                                 (2500, 6144), (1030, 16384), (3, 17000)])
@pytest.mark.parametrize("layout", [0, 1])
def test_rmsnorm_quant_parity(M, K, layout):
    log(f"rmsnorm_quant M={M} K={K} layout={layout}")
    m = fq()
    x = workloads.activations(M, K, seed=K + 11, outlier_frac=0.001)
    g = workloads.gamma(K, seed=K + 12)
    eps = 1e-6
    xb, xd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    xd.copy_(x.cuda())
    qb, q = padded(M, K, torch.uint8, 16, CANARY_U8)
    yb, y = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    G = -(-K // 128)
    s = torch.empty((G, M) if layout else (M, G), dtype=torch.float32, device="cuda")
    m.fp8q_rmsnorm_quant(xd, g.cuda(), eps, layout, q, s, y)
    torch.cuda.synchronize()
    assert canary_intact(qb, K, CANARY_U8) and canary_intact(yb, K, CANARY_BF16)
    qg, sg, yg = q.cpu().numpy(), s.cpu().numpy(), bf16_bits(y)
    if layout:
        sg = sg.T
    xh, gh = bf16_host(x), bf16_host(g)
    ref, amb = _rms_expected(xh, gh, eps, yg)
    ok = np.ones(M, bool)
    ok[amb] = False
    np.testing.assert_array_equal(yg[ok], ref["y"][ok])
    np.testing.assert_array_equal(qg[ok], ref["q"][ok])
    np.testing.assert_array_equal(sg[ok], ref["s"][ok])
    for i in amb:   # either neighbour of r, then bit-exact for that r
        r_alt = ref["r"].copy()
        r_alt[i] = ref["r_alt"][i]
        alt = oq.rmsnorm_quant(xh, gh, eps, r=r_alt)
        match = [np.array_equal(yg[i], cand["y"][i]) and np.array_equal(qg[i], cand["q"][i])
                 and np.array_equal(sg[i], cand["s"][i]) for cand in (ref, alt)]
        assert any(match), f"row {i}"


# Without the y output: row lengths at each width of the rows kernel, fewer
# rows than workgroups, a ragged share of rows per workgroup (padded rows,
# canaries).
@pytest.mark.parametrize("M,K", [(5, 2048), (64, 4096), (2500, 6144), (37, 8192), (3100, 6144),
                                 (1, 6144), (300, 2048)])
@pytest.mark.parametrize("layout", [0, 1])
def test_rmsnorm_quant_no_y_parity(M, K, layout):
    log(f"rmsnorm_quant (no y) M={M} K={K} layout={layout}")
    m = fq()
    x = workloads.activations(M, K, seed=K + 21, outlier_frac=0.001)
    g = workloads.gamma(K, seed=K + 22)
    eps = 1e-6
    xb, xd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    xd.copy_(x.cuda())
    qb, q = padded(M, K, torch.uint8, 16, CANARY_U8)
    G = -(-K // 128)
    s = torch.empty((G, M) if layout else (M, G), dtype=torch.float32, device="cuda")
    m.fp8q_rmsnorm_quant(xd, g.cuda(), eps, layout, q, s, None)
    torch.cuda.synchronize()
    assert canary_intact(qb, K, CANARY_U8)
    qg, sg = q.cpu().numpy(), s.cpu().numpy()
    if layout:
        sg = sg.T
    xh, gh = bf16_host(x), bf16_host(g)
    ref, amb = _rms_expected(xh, gh, eps, None)
    ok = np.ones(M, bool)
    ok[amb] = False
    np.testing.assert_array_equal(qg[ok], ref["q"][ok])
    np.testing.assert_array_equal(sg[ok], ref["s"][ok])
    for i in amb:   # either neighbour of r, then bit-exact for that r
        r_alt = ref["r"].copy()
        r_alt[i] = ref["r_alt"][i]
        alt = oq.rmsnorm_quant(xh, gh, eps, r=r_alt)
        match = [np.array_equal(qg[i], cand["q"][i]) and np.array_equal(sg[i], cand["s"][i])
                 for cand in (ref, alt)]
        assert any(match), f"row {i}"


@pytest.mark.parametrize("layout", [0, 1])
def test_rmsnorm_quant_full_size_sampled_rows(layout):
    # layout 1 is the bench's launch configuration
    wl = workloads.WORKLOADS["prefill_norm"]
    log(f"rmsnorm_quant full size [{wl.M},{wl.K}] layout={layout}")
    m = fq()
    d = wl.make("cpu")
    q, s = m.rmsnorm_quant(d["x"].cuda(), d["gamma"].cuda(), d["eps"], layout=layout)
    torch.cuda.synchronize()
    sg = s.cpu().numpy()
    if layout:
        sg = sg.T
    rows = np.unique(np.concatenate([[0, wl.M - 1], np.random.default_rng(1).integers(0, wl.M, 30)]))
    ref = oq.rmsnorm_quant(bf16_host(d["x"][rows]), bf16_host(d["gamma"]), d["eps"])
    ok = ~ref["ambiguous"]
    np.testing.assert_array_equal(q.cpu().numpy()[rows][ok], ref["q"][ok])
    np.testing.assert_array_equal(sg[rows][ok], ref["s"][ok])


@pytest.mark.parametrize("N,K", [(256, 512), (300, 200), (128, 1001), (1024, 7168)])
def test_weight_block_parity(N, K):
    log(f"weight_block N={N} K={K}")
    m = fq()
    w = workloads.weights(N, K, seed=N + K)
    wb, wd = padded(N, K, torch.bfloat16, 8, CANARY_BF16)
    wd.copy_(w.cuda())
    qb, q = padded(N, K, torch.uint8, 16, CANARY_U8)
    s = torch.empty(-(-N // 128), -(-K // 128), dtype=torch.float32, device="cuda")
    m.fp8q_quant_weight_block(wd, 128, 128, m.SCALE_F32, q, s)
    torch.cuda.synchronize()
    assert canary_intact(qb, K, CANARY_U8)
    qr, sr = oq.quant_weight_block(bf16_host(w))
    np.testing.assert_array_equal(s.cpu().numpy(), sr)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


def test_weight_block_full_size_sampled_block_rows():
    wl = workloads.WORKLOADS["large"]
    log(f"weight_block full size [{wl.N},{wl.K}]")
    m = fq()
    w = workloads.weights(wl.N, wl.K, wl.seed * 10 + 2)
    q, s = m.quant_weight_block(w.cuda())
    torch.cuda.synchronize()
    qg, sg = q.cpu().numpy(), s.cpu().numpy()
    for bn in (0, 77, wl.N // 128 - 1):
        rows = slice(bn * 128, (bn + 1) * 128)
        qr, sr = oq.quant_weight_block(bf16_host(w[rows]))
        np.testing.assert_array_equal(sg[bn], sr[0])
        np.testing.assert_array_equal(qg[rows], qr)


@pytest.mark.parametrize("N,K", [(300, 520), (64, 7168)])
def test_weight_tensor_parity(N, K):
    log(f"weight_tensor N={N} K={K}")
    m = fq()
    w = workloads.weights(N, K, seed=N * 3 + K)
    for _ in range(2):       # the scalar slot is reused as scratch: repeat
        q, s = m.quant_weight_tensor(w.cuda())
        torch.cuda.synchronize()
        qr, sr = oq.quant_tensor(bf16_host(w))
        assert s.cpu().numpy()[0] == sr
        np.testing.assert_array_equal(q.cpu().numpy(), qr)


@pytest.mark.parametrize("N,K", [(256, 512), (70, 200)])
def test_weight_mx_parity(N, K):
    log(f"weight_mx N={N} K={K}")
    m = fq()
    w = workloads.weights(N, K, seed=N + 2 * K, std=1.0)
    q, s = m.quant_weight_mx(w.cuda())
    torch.cuda.synchronize()
    qr, sr = oq.quant_mx(bf16_host(w))
    np.testing.assert_array_equal(s.cpu().numpy(), sr)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


def test_quantizers_deterministic():
    log("quantizer determinism")
    m = fq()
    x = workloads.activations(64, 6144, seed=99, outlier_frac=0.001).cuda()
    a = m.quant_act_group(x)
    b = m.quant_act_group(x)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
