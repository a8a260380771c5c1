"""C-ABI checks that need no GPU: exports, binding signatures, argument
validation (every case here returns before any device access), and the
exhaustive host-side proof of the quantizer's division sequence."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(fp8q_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    import fp8_block_scaled_token_amd as fq
    if not os.path.exists(fq.LIB_PATH):
        pytest.fail("libfp8q.so is not built (run __graft_entry__.build())")
    return fq.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("fp8q_quant_act_group", "fp8q_rmsnorm_quant", "fp8q_add_rmsnorm_quant", "fp8q_quant_weight_block",
              "fp8q_gemm_blockscale", "fp8q_gemm_mxfp8", "fp8q_status_string", "fp8q_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import fp8_block_scaled_token_amd as fq
    out = subprocess.run(["nm", "-D", "--defined-only", fq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(fp8q_\w+)", out))
    for n in _declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_binding_covers_every_declared_symbol():
    import fp8_block_scaled_token_amd as fq
    assert sorted(fq.SIGNATURES) == _declared_functions()


def test_abi_version_and_status_strings(lib):
    assert lib.fp8q_abi_version() == 3
    for s in range(9):
        assert len(lib.fp8q_status_string(s)) > 0
    assert lib.fp8q_status_string(99) == b"unknown status"


# fake but aligned addresses: validation must reject the call before any use
A = ctypes.c_void_p(0x100000)
B = ctypes.c_void_p(0x200000)
C = ctypes.c_void_p(0x300000)
ODD = ctypes.c_void_p(0x100008)


def test_quant_act_group_validation(lib):
    f = lib.fp8q_quant_act_group
    assert f(A, -1, 128, 128, 128, 0, 0, None, B, 128, C, None) == 2      # M < 0
    assert f(A, 4, 0, 128, 128, 0, 0, None, B, 128, C, None) == 2         # K == 0
    assert f(A, 4, 128, 128, 64, 0, 0, None, B, 128, C, None) == 3       # group 64
    assert f(A, 4, 128, 128, 128, 1, 0, None, B, 128, C, None) == 3      # UE8M0 with 128
    assert f(A, 4, 128, 128, 32, 0, 0, None, B, 128, C, None) == 3       # f32 with 32
    assert f(A, 4, 128, 128, 32, 2, 0, None, B, 128, C, None) == 3       # pow2 with 32
    assert f(A, 4, 128, 128, 128, 0, 7, None, B, 128, C, None) == 3      # bad layout
    assert f(A, 0, 128, 128, 128, 0, 0, None, None, 128, None, None) == 0  # M == 0: no-op
    assert f(None, 4, 128, 128, 128, 0, 0, None, B, 128, C, None) == 1   # null x
    assert f(A, 4, 128, 120, 128, 0, 0, None, B, 128, C, None) == 2      # ldx < K
    assert f(A, 4, 128, 132, 128, 0, 0, None, B, 128, C, None) == 4      # bf16 row not 16-B
    assert f(ODD, 4, 128, 128, 128, 0, 0, None, B, 128, C, None) == 4    # base not 16-B
    assert f(A, 4, 128, 128, 128, 0, 0, None, B, 136, C, None) == 4      # fp8 ld % 16
    assert f(A, 4, 128, 128, 128, 0, 0, None, B, 128, None, None) == 1   # null scales


def test_rmsnorm_quant_validation(lib):
    f = lib.fp8q_rmsnorm_quant
    assert f(A, B, 1e-6, -1, 128, 128, 0, B, 128, C, None, 0, None) == 2
    assert f(A, B, 0.0, 4, 128, 128, 0, B, 128, C, None, 0, None) == 7     # eps <= 0
    assert f(A, B, float("nan"), 4, 128, 128, 0, B, 128, C, None, 0, None) == 7
    assert f(A, B, 1e-6, 4, 128, 128, 5, B, 128, C, None, 0, None) == 3    # layout
    assert f(A, None, 1e-6, 4, 128, 128, 0, B, 128, C, None, 0, None) == 1  # null gamma
    assert f(A, B, 1e-6, 4, 128, 128, 0, B, 128, C, A, 100, None) == 2     # ldy < K


def test_add_rmsnorm_quant_validation(lib):
    f = lib.fp8q_add_rmsnorm_quant
    D = ctypes.c_void_p(0x400000)
    E = ctypes.c_void_p(0x500000)
    ok = (A, 128, B, 128, C, 128, D, 1e-6, 4, 128, 0, 0, None, E, 128, D, None, 0, None)

    def call(**kw):
        names = ["x", "ldx", "h", "ldh", "z", "ldz", "g", "eps", "M", "K", "fmt", "layout", "stat", "q", "ldq",
                 "s", "y", "ldy", "stream"]
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(M=-1) == 2
    assert call(K=0) == 2
    assert call(eps=0.0) == 7
    assert call(eps=float("inf")) == 7
    assert call(layout=3) == 3
    assert call(fmt=1) == 3                                               # UE8M0 bytes: not from the norm
    assert call(h=None) == 7                                              # no add, but a residual output
    assert call(M=0, x=None, h=None, z=None) == 0                         # no-op
    assert call(z=None) == 1
    assert call(g=None) == 1
    assert call(s=None) == 1                                              # dynamic exit needs scales
    assert call(ldh=120) == 2
    assert call(ldz=132) == 4
    assert call(y=E, ldy=100) == 2
    assert call(stat=ctypes.c_void_p(0x600002)) == 4                      # static scale alignment
    # residual output: x or h exactly, else disjoint
    assert call(z=ctypes.c_void_p(0x100000 + 16)) == 7                    # overlaps x
    assert call(z=ctypes.c_void_p(0x200000), ldz=256) == 7                # h's base, other stride
    assert call(z=ctypes.c_void_p(0x200000 - 256)) == 7                   # runs into h
    # accepted layouts reach the device check: see test_device_check_without_gpu


def test_requant_weight_pow2_validation(lib):
    f = lib.fp8q_requant_weight_pow2
    Q2 = ctypes.c_void_p(0x400000)
    S2 = ctypes.c_void_p(0x500000)
    assert f(A, 256, C, -1, 256, Q2, 256, S2, None) == 2
    assert f(A, 256, C, 256, 0, Q2, 256, S2, None) == 2
    assert f(A, 256, C, 0, 256, None, 256, None, None) == 0                 # N == 0
    assert f(A, 256, None, 256, 256, Q2, 256, S2, None) == 1
    assert f(A, 256, C, 256, 256, Q2, 256, None, None) == 1
    assert f(A, 200, C, 256, 256, Q2, 256, S2, None) == 2                    # ldi < K
    assert f(A, 256, C, 256, 256, Q2, 264, S2, None) == 4                    # ldo % 16
    assert f(A, 256, ctypes.c_void_p(0x300002), 256, 256, Q2, 256, S2, None) == 4
    assert f(A, 256, C, 256, 256, ctypes.c_void_p(0x100000 + 256), 256, S2, None) == 7   # overlaps q_in
    assert f(A, 256, C, 256, 256, A, 512, S2, None) == 7                     # q_in's base, other stride
    assert f(A, 256, C, 256, 256, Q2, 256, ctypes.c_void_p(0x300000 + 4), None) == 7     # overlaps s_in
    assert f(A, 256, C, 256, 256, ctypes.c_void_p(0x300000), 256, S2, None) == 7        # q_out over s_in
    assert f(A, 256, C, 256, 256, Q2, 256, ctypes.c_void_p(0x100000), None) == 7        # s_out over q_in


def test_gemm_splitk_validation(lib):
    f = lib.fp8q_gemm_blockscale_splitk
    W = ctypes.c_void_p(0x800000)
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, -1, 256, 128, 0, W, 1 << 20, None) == 2
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 5, W, 1 << 20, None) == 3
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 0, None, 64, None) == 1   # bytes, no buffer
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 0, ctypes.c_void_p(0x800002), 64, None) == 4
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, 0, 256, 128, 0, W, 64, None) == 0      # M == 0
    assert lib.fp8q_gemm_splitk_workspace_size(0, 256, 128) == 0


def test_gemm_grouped_validation(lib):
    f = lib.fp8q_gemm_grouped_blockscale
    O = ctypes.c_void_p(0x600000)
    ok = [A, 256, C, 0, O, 4, B, 256, 256 * 256, C, 0, ctypes.c_void_p(0x700000), 256, 100, 256, 256, 0, None]

    def call(**kw):
        names = ["a", "lda", "sa", "layout", "off", "E", "w", "ldw", "wstride", "sw", "shard", "y", "ldy", "M", "N",
                 "K", "gran", "stream"]
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(M=-1) == 2
    assert call(E=0) == 2 and call(E=1025) == 2
    assert call(shard=-64) == 2
    assert call(gran=1) == 3                                   # per-tensor is not grouped
    assert call(layout=2) == 3
    assert call(K=200, lda=208, ldw=208) == 3                  # K % 128
    assert call(shard=100) == 3                                # not a multiple of 64
    assert call(shard=192) == 3                                # does not divide N = 256
    assert call(M=0) == 0
    assert call(off=None) == 1
    assert call(sw=None) == 1
    assert call(off=ctypes.c_void_p(0x600002)) == 4
    assert call(wstride=256 * 255) == 2                        # experts overlap
    assert call(wstride=256 * 256 + 8) == 4
    assert call(ldy=200) == 2


def test_quant_weight_block_validation(lib):
    f = lib.fp8q_quant_weight_block
    assert f(A, 256, 256, 256, 64, 64, 0, B, 256, C, None) == 3          # 64x64 blocks
    assert f(A, 256, 256, 256, 1, 32, 0, B, 256, C, None) == 3           # MX block, f32
    assert f(A, 256, 256, 256, 32, 32, 1, B, 256, C, None) == 3          # MX must be 1x32
    assert f(A, 256, 256, 256, 1, 32, 2, B, 256, C, None) == 3           # pow2 needs 128x128
    assert f(A, 256, 256, 256, 128, 128, 0, B, 256, None, None) == 1
    assert f(A, -2, 256, 256, 128, 128, 0, B, 256, C, None) == 2


def test_gemm_validation(lib):
    g = lib.fp8q_gemm_blockscale
    assert g(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 0, 0, None) == 2     # K == 0
    assert g(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 9, None) == 3   # gran
    assert g(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 3, None) == 3
    assert g(A, 128, C, 0, B, 128, C, None, C, 256, 0, 256, 128, 0, None) == 0   # M == 0
    assert g(A, 120, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 0, None) == 2   # lda < K
    assert g(A, 128, None, 0, B, 128, C, None, C, 256, 4, 256, 128, 0, None) == 1
    assert g(A, 128, C, 0, B, 128, C, None, C, 252, 4, 256, 128, 0, None) == 2   # ldy < N
    assert g(A, 128, C, 0, B, 128, C, None, C, 260, 4, 260, 128, 0, None) == 4   # ldy % 8
    m = lib.fp8q_gemm_mxfp8
    assert m(A, 128, C, B, 128, C, 0, None, C, 256, -1, 256, 128, None) == 2
    assert m(A, 128, None, B, 128, C, 0, None, C, 256, 4, 256, 128, None) == 1
    assert m(A, 128, C, B, 128, C, 2, None, C, 256, 128, 256, 128, None) == 3        # layout
    assert m(A, 128, C, B, 128, C, 1, None, C, 256, 64, 256, 128, None) == 3         # column-major needs M > 64
    assert m(A, 128, C, B, 128, C, 1, None, C, 256, 130, 256, 128, None) == 3        # ... and M % 4 == 0
    assert m(A, 200, C, B, 200, C, 1, None, C, 256, 128, 256, 200, None) == 3        # ... and K % 128 == 0
    assert m(A, 128, ctypes.c_void_p(0x300001), B, 128, C, 1, None, C, 256, 128, 256, 128, None) == 4


def test_device_check_without_gpu(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid-looking fake pointers must never reach a launch")
    f = lib.fp8q_quant_act_group
    assert f(A, 4, 128, 128, 128, 0, 0, None, B, 128, C, None) == 5
    # accepted residual outputs (in place on x or h, or just past x) and the
    # static exit with an unused layout pass validation and stop here
    g = lib.fp8q_add_rmsnorm_quant
    E = ctypes.c_void_p(0x500000)
    for z in (A, B, ctypes.c_void_p(0x100000 + 128 * 2 * 4)):
        assert g(A, 128, B, 128, z, 128, C, 1e-6, 4, 128, 0, 0, None, E, 128, C, None, 0, None) == 5
    assert g(A, 128, B, 128, A, 128, C, 1e-6, 4, 128, 9, 3, ctypes.c_void_p(0x600000), E, 128, None, None, 0,
             None) == 5
    assert g(A, 128, None, 0, None, 0, C, 1e-6, 4, 128, 2, 1, None, E, 128, C, None, 0, None) == 5  # no add, pow2
    # power-of-two formats are accepted by the quantizers, the requant and the GEMM
    assert lib.fp8q_quant_act_group(A, 4, 128, 128, 128, 2, 0, None, B, 128, C, None) == 5
    assert lib.fp8q_quant_weight_block(A, 256, 256, 256, 128, 128, 2, B, 256, C, None) == 5
    assert lib.fp8q_requant_weight_pow2(A, 256, C, 256, 256, A, 256, C, None) == 5          # in place
    assert lib.fp8q_gemm_blockscale(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 2, None) == 5
    assert lib.fp8q_gemm_blockscale_splitk(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 0, None, 0, None) == 5
    assert lib.fp8q_gemm_splitk_workspace_size(32, 2048, 7168) == 0          # no device: no split
    # the grouped GEMM with shards (and the power-of-two format)
    assert lib.fp8q_gemm_grouped_blockscale(A, 256, C, 1, ctypes.c_void_p(0x600000), 4, B, 256, 512 * 256, C, 256,
                                            ctypes.c_void_p(0x700000), 512, 100, 512, 256, 2, None) == 5


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_quantizer_division_sequence_exhaustive(tmp_path):
    src = os.path.join(ROOT, "tests", "host", "div_by_scale_exhaustive.c")
    exe = str(tmp_path / "divchk")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", "-o", exe, src, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "fatal=0" in r.stdout


def test_plan_override_validation(lib):
    f = lib.fp8q_set_plan_override
    try:
        assert f(2, 0, 1, -1, -1, 0) == 7 and f(-2, 0, 1, -1, -1, 0) == 7     # gemm_cfg
        assert f(-1, -1, 1, -1, -1, 0) == 7                                    # gemm_slots
        assert f(-1, 0, 2, -1, -1, 0) == 7 and f(-1, 0, 1, 2, -1, 0) == 7      # split, decode_wide
        assert f(-1, 0, 1, -1, -2, 0) == 7                                     # wait limit
        assert f(-1, 0, 1, -1, -1, -1) == 7 and f(-1, 0, 1, -1, -1, 10001) == 7   # publish delay
        assert f(1, 64, 0, 1, 0, 5) == 0 and f(0, 0, 1, 0, -1, 0) == 0
    finally:
        assert f(-1, 0, 1, -1, -1, 0) == 0


def test_library_reads_no_environment():
    # the launch plans come only from arguments and fp8q_set_plan_override
    src = os.path.join(ROOT, "fp8_block_scaled_token_amd", "csrc")
    for name in os.listdir(src):
        text = open(os.path.join(src, name)).read()
        assert "getenv" not in text and "secure_getenv" not in text, name


def test_gemm_splitk_noalloc_validation(lib):
    f = lib.fp8q_gemm_blockscale_splitk_noalloc
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, -1, 256, 128, 0, None) == 2        # M < 0
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 5, None) == 3         # gran
    assert f(A, 128, C, 2, B, 128, C, None, C, 256, 4, 256, 128, 0, None) == 3         # layout
    assert f(A, 128, None, 0, B, 128, C, None, C, 256, 4, 256, 128, 0, None) == 1      # no scales
    assert f(A, 128, ctypes.c_void_p(0x300002), 0, B, 128, C, None, C, 256, 4, 256, 128, 0, None) == 4
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, 0, 256, 128, 0, None) == 0         # M == 0
    assert f(A, 128, C, 0, B, 128, C, None, C, 256, 4, 256, 128, 0, None) == 5         # no device here
    assert lib.fp8q_status_string(8).startswith(b"problem needs more split-K scratch")
