"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the fused RMSNorm quantizer and the split-tail prefill GEMM (whose flags a
replay reuses with the same launch value), and every other entry point.  Every replay, with the program's
own eager work and synchronizations between replays, must give the eager
result bit for bit (all kernels here are deterministic)."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import bf16_bits, log

pytestmark = pytest.mark.gpu


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def test_graph_replay_of_norm_quant_and_split_gemm():
    m = fq()
    M, N, K = 2304, 8192, 4096                      # 288 tiles: a split tail on 256 CUs
    log(f"graph replay M={M} N={N} K={K}")
    x = workloads.activations(M, K, seed=3, outlier_frac=0.001).cuda()
    g = workloads.gamma(K, seed=4).cuda()
    w = workloads.weights(N, K, seed=5).cuda()
    qw, sw = m.quant_weight_block(w)
    nbytes = m.fp8q_gemm_splitk_workspace_size(M, N, K)
    assert nbytes > 0
    ws = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    q = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    s = torch.empty(K // 128, M, dtype=torch.float32, device="cuda")
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")

    def step():
        m.fp8q_rmsnorm_quant(x, g, 1e-6, m.COL_MAJOR, q, s)
        m.fp8q_gemm_blockscale_splitk(q, s, m.COL_MAJOR, qw, sw, None, y, m.GRAN_BLOCK128, ws)

    step()
    torch.cuda.synchronize()
    y_eager, q_eager = bf16_bits(y), q.cpu().numpy()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                   # warm up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    other = torch.empty_like(y)
    for rep in range(4):
        y.zero_()
        q.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q.cpu().numpy(), q_eager, err_msg=f"replay {rep}: codes")
        np.testing.assert_array_equal(bf16_bits(y), y_eager, err_msg=f"replay {rep}: output")
        # the program's own eager work between replays, on the same workspace
        m.fp8q_gemm_blockscale_splitk(q, s, m.COL_MAJOR, qw, sw, None, other, m.GRAN_BLOCK128, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_bits(other), y_eager, err_msg=f"eager after replay {rep}")


def test_graph_replay_of_every_entry_point():
    """The other entry points captured together (as the bench captures its
    timing loops): group, MX and static quantizers, the split decode GEMM
    with its reduction, the MoE grouped GEMM, the MX and per-tensor GEMMs.
    Every replay must give the eager bits."""
    m = fq()
    dev = "cuda"
    # decode split-K (112 K blocks: split) behind the group quantizer
    xd = workloads.activations(32, 14336, seed=11, outlier_frac=0.001).to(dev)
    wd = workloads.weights(2048, 14336, seed=12).to(dev)
    qwd, swd = m.quant_weight_block(wd)
    qd = torch.empty(32, 14336, dtype=torch.uint8, device=dev)
    sd = torch.empty(112, 32, dtype=torch.float32, device=dev)
    nbytes = m.fp8q_gemm_splitk_workspace_size(32, 2048, 14336)
    assert nbytes > 0
    wsd = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)
    yd = torch.empty(32, 2048, dtype=torch.bfloat16, device=dev)
    # MX, column-major scale bytes (the fast kernel's layout)
    xm = workloads.activations(256, 2048, seed=13).to(dev)
    qwm, swm = m.quant_act_mx(workloads.weights(512, 2048, seed=14).to(dev), layout=m.COL_MAJOR)
    qm = torch.empty(256, 2048, dtype=torch.uint8, device=dev)
    sm = torch.empty(64, 256, dtype=torch.uint8, device=dev)
    ym = torch.empty(256, 512, dtype=torch.bfloat16, device=dev)
    # static per-tensor activations and a per-tensor weight
    xs = workloads.activations(128, 1024, seed=15).to(dev)
    sx = torch.tensor([float(xs.float().abs().max()) / 448.0], dtype=torch.float32, device=dev)
    qws, sws = m.quant_weight_tensor(workloads.weights(384, 1024, seed=16).to(dev))
    qs = torch.empty(128, 1024, dtype=torch.uint8, device=dev)
    ys = torch.empty(128, 384, dtype=torch.bfloat16, device=dev)
    # MoE: 4 experts over 420 expert-sorted rows
    E, N, K = 4, 512, 1024
    offs = torch.tensor([0, 100, 250, 300, 420], dtype=torch.int32, device=dev)
    xe = workloads.activations(420, K, seed=17).to(dev)
    qwe = torch.empty(E, N, K, dtype=torch.uint8, device=dev)
    swe = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=dev)
    for e in range(E):
        m.fp8q_quant_weight_block(workloads.weights(N, K, seed=20 + e).to(dev), 128, 128, m.SCALE_F32, qwe[e], swe[e])
    qe = torch.empty(420, K, dtype=torch.uint8, device=dev)
    se = torch.empty(K // 128, 420, dtype=torch.float32, device=dev)
    ye = torch.empty(420, N, dtype=torch.bfloat16, device=dev)

    def run():
        m.fp8q_quant_act_group(xd, 128, m.SCALE_F32, m.COL_MAJOR, None, qd, sd)
        m.fp8q_gemm_blockscale_splitk(qd, sd, m.COL_MAJOR, qwd, swd, None, yd, m.GRAN_BLOCK128, wsd)
        m.fp8q_quant_act_group(xm, 32, m.SCALE_UE8M0, m.COL_MAJOR, None, qm, sm)
        m.fp8q_gemm_mxfp8(qm, sm, qwm, swm, None, ym, m.COL_MAJOR)
        m.fp8q_quant_act_group(xs, 128, m.SCALE_F32, m.ROW_MAJOR, sx, qs, None)
        m.fp8q_gemm_blockscale(qs, sx, m.ROW_MAJOR, qws, sws, None, ys, m.GRAN_PER_TENSOR)
        m.fp8q_quant_act_group(xe, 128, m.SCALE_F32, m.COL_MAJOR, None, qe, se)
        m.fp8q_gemm_grouped_blockscale(qe, se, m.COL_MAJOR, offs, qwe, swe, ye, 0, m.GRAN_BLOCK128)

    outs = [qd, sd, yd, qm, sm, ym, qs, ys, qe, se, ye]

    def bits():
        torch.cuda.synchronize()
        return [o.view(torch.uint8).cpu().numpy().copy() for o in outs]

    log("graph replay of every entry point")
    run()
    eager = bits()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        for i, (a, b) in enumerate(zip(bits(), eager)):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}: output {i}")
        run()                                          # eager work between replays
        for i, (a, b) in enumerate(zip(bits(), eager)):
            np.testing.assert_array_equal(a, b, err_msg=f"eager after replay {rep}: output {i}")
