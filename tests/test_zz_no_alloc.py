"""The allocation-free split-K GEMM entry point (fp8q_gemm_blockscale_splitk_noalloc),
called through the C ABI, against the entry point with a caller workspace
(fp8q_gemm_blockscale_splitk): the same kernels and split choice, so the
same bits.  Two calls in a row, the second with a smaller problem (the
library's scratch keeps the first call's contents), for a prefill shape
whose leftover tiles meet in the scratch and a decode shape whose K
segments' partials go there; a problem that needs more scratch than the
entry holds is refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_helpers import bf16_bits, bf16_host, check_gemm_rows, log

pytestmark = pytest.mark.gpu


def fq():
    import fp8_block_scaled_token_amd as m
    return m


def _problem(M, N, K, seed):
    x = bf16_host(workloads.activations(M, K, seed, 0.001))
    w = bf16_host(workloads.weights(N, K, seed + 1))
    qa, sa = oq.quant_group(x)
    qw, sw = oq.quant_weight_block(w)
    dev = dict(a=torch.from_numpy(qa).cuda(), sa=torch.from_numpy(np.ascontiguousarray(sa.T)).cuda(),
               w=torch.from_numpy(qw).cuda(), sw=torch.from_numpy(sw).cuda())
    return (qa, sa, qw, sw), dev


def _noalloc_raw(d, y, gran=0):
    """One call through ctypes with raw pointers: the C ABI itself."""
    lib = fq().load_library()
    M, K = d["a"].shape
    N = d["w"].shape[0]
    return lib.fp8q_gemm_blockscale_splitk_noalloc(
        ctypes.c_void_p(d["a"].data_ptr()), K, ctypes.c_void_p(d["sa"].data_ptr()), 1,
        ctypes.c_void_p(d["w"].data_ptr()), K, ctypes.c_void_p(d["sw"].data_ptr()), None,
        ctypes.c_void_p(y.data_ptr()), N, M, N, K, gran,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _with_workspace(d, y):
    m = fq()
    M, K = d["a"].shape
    N = d["w"].shape[0]
    nbytes = m.fp8q_gemm_splitk_workspace_size(M, N, K)
    ws = torch.full((max(nbytes, 8) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    m.fp8q_gemm_blockscale_splitk(d["a"], d["sa"], 1, d["w"], d["sw"], None, y, m.GRAN_BLOCK128, ws)
    return nbytes


def test_noalloc_equals_workspace_entry_on_two_calls():
    m = fq()
    assert m.abi_version() == 3
    cases = [(2304, 8192, 4096, 3), (32, 2048, 28672, 9)]     # prefill tail split, then a smaller decode split
    for M, N, K, seed in cases:
        log(f"noalloc M={M} N={N} K={K}")
        host, d = _problem(M, N, K, seed)
        y_ws = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        nbytes = _with_workspace(d, y_ws)
        assert 0 < nbytes <= (33 << 20)
        y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert _noalloc_raw(d, y_na) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_bits(y_na), bf16_bits(y_ws))
        rows = np.unique(np.r_[0, M - 1, np.random.default_rng(seed).integers(0, M, 6)])
        yr = og.gemm_blockscale(*host, rows=rows)[0]
        check_gemm_rows(bf16_bits(y_na)[rows], yr, f"noalloc M={M} N={N} K={K}", 1e-2)


def test_noalloc_refuses_problems_beyond_its_scratch(plan):
    m = fq()
    M, N, K = 4096, 11264, 4096
    # planned for 512 CUs: 704 tiles leave 192 leftover tiles of 256 KB partials
    plan(gemm_slots=512)
    need = m.fp8q_gemm_splitk_workspace_size(M, N, K)
    log(f"noalloc refusal: needs {need} bytes")
    assert need > (33 << 20)
    d = dict(a=torch.zeros(M, K, dtype=torch.uint8, device="cuda"),
             sa=torch.ones(K // 128, M, dtype=torch.float32, device="cuda"),
             w=torch.zeros(N, K, dtype=torch.uint8, device="cuda"),
             sw=torch.ones(N // 128, K // 128, dtype=torch.float32, device="cuda"))
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    assert _noalloc_raw(d, y) == 8
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "nothing may be launched"
