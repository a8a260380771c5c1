"""GPU parity of the fused residual add -> RMSNorm -> quantization entry point
against the CPU oracle: the updated residual stream, the normalized rows, the
codes and the group scales bit for bit (rows whose fp32 RMS factor is a near
tie accept either neighbour, then match bit for bit for it).  Both exits
(group-128 with either scale layout, static per-tensor), in place on the
stream and into a separate buffer, with and without the y copy, on row
lengths that cover every rows-kernel width, ragged rows and rows longer than
the one-read limit."""
import numpy as np
import pytest
import torch

import workloads
from oracle import bf16 as obf16
from oracle import quant as oq
from tests.gpu_helpers import CANARY_BF16, CANARY_U8, bf16_bits, bf16_host, canary_intact, log, padded

pytestmark = pytest.mark.gpu

EPS = 1e-6
SMALL = [(16, 512), (5, 520), (64, 6144), (3, 7168), (4, 9000), (2, 1001), (1, 6144), (37, 8192),
         (9, 12288), (3, 17000)]
LARGE = [(2500, 6144), (1030, 16384)]


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _inputs(M, K, seed):
    x = workloads.activations(M, K, seed=seed, outlier_frac=0.001)
    # a sublayer output: smaller, with its own outlier channels
    h = (workloads.activations(M, K, seed=seed + 1, outlier_frac=0.001).float() * 0.25).to(torch.bfloat16)
    g = workloads.gamma(K, seed=seed + 2)
    return x, h, g


def _check(M, K, mode, inplace, with_y, seed):
    m = fq()
    x, h, g = _inputs(M, K, seed)
    xb, xd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    xd.copy_(x.cuda())
    hb, hd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    hd.copy_(h.cuda())
    if inplace:
        zb, zd = xb, xd
    else:
        zb, zd = padded(M, K, torch.bfloat16, 8, CANARY_BF16)
    qb, q = padded(M, K, torch.uint8, 16, CANARY_U8)
    yb, y = padded(M, K, torch.bfloat16, 8, CANARY_BF16) if with_y else (None, None)
    G = -(-K // 128)
    static = mode == "static"
    layout = 1 if mode == "group_col" else 0
    sx = np.float32(0.0137)
    sd = torch.tensor([sx], dtype=torch.float32, device="cuda") if static else None
    s = None if static else torch.empty((G, M) if layout else (M, G), dtype=torch.float32, device="cuda")
    m.fp8q_add_rmsnorm_quant(xd, hd, zd, g.cuda(), EPS, m.SCALE_F32, layout, sd, q, s, y)
    torch.cuda.synchronize()
    assert canary_intact(zb, K, CANARY_BF16) and canary_intact(qb, K, CANARY_U8)
    assert canary_intact(hb, K, CANARY_BF16)
    if not inplace:
        assert canary_intact(xb, K, CANARY_BF16)
        np.testing.assert_array_equal(bf16_bits(xd), bf16_bits(x))      # x untouched
    np.testing.assert_array_equal(bf16_bits(hd), bf16_bits(h))          # h untouched
    if with_y:
        assert canary_intact(yb, K, CANARY_BF16)
    zg, qg = bf16_bits(zd), q.cpu().numpy()
    yg = bf16_bits(y) if with_y else None
    sg = None
    if not static:
        sg = s.cpu().numpy()
        if layout:
            sg = sg.T
    xh, hh, gh = bf16_host(x), bf16_host(h), bf16_host(g)
    ref = oq.add_rmsnorm_quant(xh, hh, gh, EPS, static_scale=sx if static else None)
    np.testing.assert_array_equal(zg, ref["z"])
    amb = np.flatnonzero(ref["ambiguous"])
    if amb.size:
        log(f"  near-tie rows: {amb.tolist()}")
    ok = np.ones(M, bool)
    ok[amb] = False

    def same(cand, rows):
        eq = np.array_equal(qg[rows], cand["q"][rows])
        if with_y:
            eq = eq and np.array_equal(yg[rows], cand["y"][rows])
        if not static:
            eq = eq and np.array_equal(sg[rows], cand["s"][rows])
        return eq

    np.testing.assert_array_equal(qg[ok], ref["q"][ok])
    if with_y:
        np.testing.assert_array_equal(yg[ok], ref["y"][ok])
    if not static:
        np.testing.assert_array_equal(sg[ok], ref["s"][ok])
    for i in amb:
        r_alt = ref["r"].copy()
        r_alt[i] = ref["r_alt"][i]
        alt = oq.add_rmsnorm_quant(xh, hh, gh, EPS, static_scale=sx if static else None, r=r_alt)
        assert same(ref, [i]) or same(alt, [i]), f"row {i}"
    if static:
        assert np.any((qg & 0x7F) == 0x7E), "the static scale should saturate some outliers"


@pytest.mark.parametrize("M,K", SMALL)
@pytest.mark.parametrize("mode", ["group_row", "group_col", "static"])
@pytest.mark.parametrize("inplace", [True, False])
def test_add_rmsnorm_quant_parity(M, K, mode, inplace):
    log(f"add_rmsnorm_quant M={M} K={K} mode={mode} inplace={inplace}")
    _check(M, K, mode, inplace, with_y=not inplace, seed=K + 31)


@pytest.mark.parametrize("M,K", LARGE)
@pytest.mark.parametrize("mode", ["group_col", "static"])
def test_add_rmsnorm_quant_many_rows(M, K, mode):
    log(f"add_rmsnorm_quant many rows M={M} K={K} mode={mode}")
    _check(M, K, mode, inplace=True, with_y=False, seed=K + 41)


def test_add_rmsnorm_quant_in_place_on_h():
    # residual_out may be h itself
    log("add_rmsnorm_quant residual_out = h")
    m = fq()
    M, K = 40, 6144
    x, h, g = _inputs(M, K, 77)
    xd, hd = x.cuda(), h.cuda()
    q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    s = torch.empty(M, K // 128, dtype=torch.float32, device="cuda")
    m.fp8q_add_rmsnorm_quant(xd, hd, hd, g.cuda(), EPS, m.SCALE_F32, 0, None, q, s)
    torch.cuda.synchronize()
    ref = oq.add_rmsnorm_quant(bf16_host(x), bf16_host(h), bf16_host(g), EPS)
    np.testing.assert_array_equal(bf16_bits(hd), ref["z"])
    ok = ~ref["ambiguous"]
    np.testing.assert_array_equal(q.cpu().numpy()[ok], ref["q"][ok])
    np.testing.assert_array_equal(s.cpu().numpy()[ok], ref["s"][ok])


def test_add_rmsnorm_quant_equals_add_then_rmsnorm_quant():
    # fusion changes no bits: the GPU's own unfused sequence gives the same bytes
    log("add_rmsnorm_quant vs add + rmsnorm_quant")
    m = fq()
    M, K = 300, 7168
    x, h, g = _inputs(M, K, 91)
    gd = g.cuda()
    xd = x.cuda()
    q1, s1, y1 = m.add_rmsnorm_quant(xd, h.cuda(), gd, EPS, return_y=True)
    z_ref = torch.from_numpy(oq.residual_add(bf16_host(x), bf16_host(h)).view(np.int16)).view(torch.bfloat16)
    q2, s2, y2 = m.rmsnorm_quant(z_ref.cuda(), gd, EPS, return_y=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(xd), bf16_bits(z_ref))
    np.testing.assert_array_equal(q1.cpu().numpy(), q2.cpu().numpy())
    np.testing.assert_array_equal(s1.cpu().numpy(), s2.cpu().numpy())
    np.testing.assert_array_equal(bf16_bits(y1), bf16_bits(y2))


def test_add_rmsnorm_quant_full_size_sampled_rows():
    # the prefill shape [4096, 6144] in the bench's launch configuration
    wl = workloads.WORKLOADS["prefill_norm"]
    log(f"add_rmsnorm_quant full size [{wl.M},{wl.K}]")
    m = fq()
    d = wl.make("cpu")
    h = (workloads.activations(wl.M, wl.K, seed=5, outlier_frac=0.001).float() * 0.25).to(torch.bfloat16)
    xd = d["x"].cuda()
    q, s = m.add_rmsnorm_quant(xd, h.cuda(), d["gamma"].cuda(), d["eps"], layout=m.COL_MAJOR)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, wl.M - 1], np.random.default_rng(2).integers(0, wl.M, 30)]))
    ref = oq.add_rmsnorm_quant(bf16_host(d["x"][rows]), bf16_host(h[rows]), bf16_host(d["gamma"]), d["eps"])
    np.testing.assert_array_equal(bf16_bits(xd)[rows], ref["z"])
    ok = ~ref["ambiguous"]
    np.testing.assert_array_equal(q.cpu().numpy()[rows][ok], ref["q"][ok])
    np.testing.assert_array_equal(s.cpu().numpy().T[rows][ok], ref["s"][ok])


def test_add_rmsnorm_quant_deterministic():
    m = fq()
    M, K = 512, 6144
    x, h, g = _inputs(M, K, 99)
    outs = []
    for _ in range(2):
        xd = x.cuda()
        q, s = m.add_rmsnorm_quant(xd, h.cuda(), g.cuda(), EPS)
        torch.cuda.synchronize()
        outs.append((bf16_bits(xd), q.cpu().numpy(), s.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)
