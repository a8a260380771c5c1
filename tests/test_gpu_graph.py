"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the fused RMSNorm quantizer and the split-tail prefill GEMM (whose flags a
replay reuses with the same launch value).  Every replay, with the program's
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
