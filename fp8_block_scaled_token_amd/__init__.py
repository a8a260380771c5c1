"""fp8_block_scaled_token_amd -- Python binding of libfp8q (MI355X / gfx950).

Argument marshalling only: every computation runs in the HIP kernels of
libfp8q.so, reached through its C ABI (include/fp8q.h).  torch supplies device
memory and the current stream.  There is no fallback: if the library is
missing or the device is not gfx950 the calls raise.

Functions named ``fp8q_*`` mirror the C entry points one to one (tensors in
place of pointers, sizes read from the tensors).  The short-named helpers
(``quant_act_group`` ...) allocate the outputs and call them.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "load_library", "FP8QError", "abi_version", "fp8q_set_plan_override", "plan_override",
    "fp8q_quant_act_group", "fp8q_rmsnorm_quant", "fp8q_add_rmsnorm_quant", "fp8q_quant_weight_block",
    "fp8q_requant_weight_pow2", "fp8q_gemm_blockscale", "fp8q_gemm_blockscale_splitk",
    "fp8q_gemm_splitk_workspace_size", "fp8q_gemm_blockscale_splitk_noalloc", "fp8q_gemm_grouped_blockscale",
    "fp8q_gemm_mxfp8",
    "quant_act_group", "quant_act_group_pow2", "rmsnorm_quant_pow2", "quant_act_static", "quant_act_mx", "rmsnorm_quant", "add_rmsnorm_quant",
    "quant_weight_block", "quant_weight_block_pow2", "requant_weight_pow2", "quant_weight_mx", "quant_weight_tensor",
    "gemm_blockscale", "gemm_blockscale_pow2", "gemm_blockscale_splitk", "gemm_grouped_blockscale",
    "gemm_pertensor", "gemm_mxfp8",
    "SCALE_F32", "SCALE_UE8M0", "SCALE_F32_POW2", "ROW_MAJOR", "COL_MAJOR", "GRAN_BLOCK128", "GRAN_PER_TENSOR",
    "GRAN_BLOCK128_POW2",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8q.so")

SCALE_F32, SCALE_UE8M0, SCALE_F32_POW2 = 0, 1, 2
ROW_MAJOR, COL_MAJOR = 0, 1
GRAN_BLOCK128, GRAN_PER_TENSOR, GRAN_BLOCK128_POW2 = 0, 1, 2

_STATUS = {0: "ok", 1: "null", 2: "shape", 3: "unsupported", 4: "misaligned",
           5: "device", 6: "launch", 7: "value", 8: "scratch"}

#: exported symbol -> (restype, argtypes); mirrors include/fp8q.h
_P, _I64, _I32, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
SIGNATURES = {
    "fp8q_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8q_abi_version": (ctypes.c_int, []),
    "fp8q_set_plan_override": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "fp8q_quant_act_group": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _I64, _P, _P]),
    "fp8q_rmsnorm_quant": (ctypes.c_int, [_P, _P, _F, _I64, _I64, _I64, _I32, _P, _I64, _P, _P, _I64, _P]),
    "fp8q_add_rmsnorm_quant": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _P, _F, _I64, _I64, _I32, _I32, _P, _P,
                                              _I64, _P, _P, _I64, _P]),
    "fp8q_requant_weight_pow2": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _P, _I64, _P, _P]),
    "fp8q_quant_weight_block": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _I64, _P, _P]),
    "fp8q_gemm_blockscale": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P]),
    "fp8q_gemm_splitk_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "fp8q_gemm_blockscale_splitk": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64,
                                                   _I32, _P, ctypes.c_size_t, _P]),
    "fp8q_gemm_blockscale_splitk_noalloc": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _I64, _P, _P, _P, _I64, _I64,
                                                           _I64, _I64, _I32, _P]),
    "fp8q_gemm_grouped_blockscale": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _I32, _P, _I64, _I64, _P, _I64, _P, _I64,
                                                    _I64, _I64, _I64, _I32, _P]),
    "fp8q_gemm_mxfp8": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _P, _I32, _P, _P, _I64, _I64, _I64, _I64, _P]),
}

_lib: Optional[ctypes.CDLL] = None


class FP8QError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = load_library().fp8q_status_string(status).decode()
        super().__init__(f"{what}: {msg} (status {status}, {_STATUS.get(status, '?')})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp8q.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} not found: build it with `python -m fp8_block_scaled_token_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def abi_version() -> int:
    return load_library().fp8q_abi_version()


def fp8q_set_plan_override(gemm_cfg: int = -1, gemm_slots: int = 0, gemm_split: int = 1,
                           decode_wide: int = -1, split_wait_limit: int = -1,
                           split_publish_delay: int = 0) -> None:
    """Force GEMM launch plans process-wide (defaults: automatic plans)."""
    _check(load_library().fp8q_set_plan_override(gemm_cfg, gemm_slots, gemm_split, decode_wide,
                                                 split_wait_limit, split_publish_delay),
           "fp8q_set_plan_override")


@contextlib.contextmanager
def plan_override(**kw):
    """fp8q_set_plan_override(**kw) for the duration of a with-block."""
    fp8q_set_plan_override(**kw)
    try:
        yield
    finally:
        fp8q_set_plan_override()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise FP8QError(status, what)


def _rows(t: torch.Tensor, dtype: torch.dtype, name: str):
    """(rows, K, ld) of a row-major 2-D tensor with unit column stride."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D row-major tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.size(0), t.size(1), t.stride(0)


def _u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


# --------------------------------------------------------------------------
# one-to-one mirrors of the C entry points


def fp8q_quant_act_group(x, group_size, fmt, layout, static_scale, q, scales, stream=None):
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    q = _u8(q)
    Mq, Kq, ldq = _rows(q, torch.uint8, "q")
    if (Mq, Kq) != (M, K):
        raise ValueError("q shape must match x")
    _check(load_library().fp8q_quant_act_group(_ptr(x), M, K, ldx, group_size, fmt, layout,
                                               _ptr(static_scale), _ptr(q), ldq, _ptr(scales),
                                               _stream(stream)), "fp8q_quant_act_group")


def fp8q_rmsnorm_quant(x, gamma, eps, layout, q, scales, y_out=None, stream=None):
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    q = _u8(q)
    _, _, ldq = _rows(q, torch.uint8, "q")
    ldy = 0
    if y_out is not None:
        _, _, ldy = _rows(y_out, torch.bfloat16, "y_out")
    if gamma.dtype != torch.bfloat16 or gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous bf16 tensor of K elements")
    _check(load_library().fp8q_rmsnorm_quant(_ptr(x), _ptr(gamma), float(eps), M, K, ldx, layout,
                                             _ptr(q), ldq, _ptr(scales), _ptr(y_out), ldy,
                                             _stream(stream)), "fp8q_rmsnorm_quant")


def fp8q_add_rmsnorm_quant(x, h, residual_out, gamma, eps, fmt, layout, static_scale, q, scales, y_out=None,
                           stream=None):
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    ldh = ldr = 0
    if h is not None:
        Mh, Kh, ldh = _rows(h, torch.bfloat16, "h")
        Mr, Kr, ldr = _rows(residual_out, torch.bfloat16, "residual_out")
        if (Mh, Kh) != (M, K) or (Mr, Kr) != (M, K):
            raise ValueError("h and residual_out must have the shape of x")
    q = _u8(q)
    _, _, ldq = _rows(q, torch.uint8, "q")
    ldy = 0
    if y_out is not None:
        _, _, ldy = _rows(y_out, torch.bfloat16, "y_out")
    if gamma.dtype != torch.bfloat16 or gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous bf16 tensor of K elements")
    _check(load_library().fp8q_add_rmsnorm_quant(_ptr(x), ldx, _ptr(h), ldh, _ptr(residual_out), ldr,
                                                 _ptr(gamma), float(eps), M, K, fmt, layout, _ptr(static_scale),
                                                 _ptr(q), ldq, _ptr(scales), _ptr(y_out), ldy,
                                                 _stream(stream)), "fp8q_add_rmsnorm_quant")


def fp8q_requant_weight_pow2(q_in, s_in, q_out, s_out, stream=None):
    q_in, q_out = _u8(q_in), _u8(q_out)
    N, K, ldi = _rows(q_in, torch.uint8, "q_in")
    No, Ko, ldo = _rows(q_out, torch.uint8, "q_out")
    if (No, Ko) != (N, K):
        raise ValueError("q_out must have the shape of q_in")
    shape = (_cdiv(N, 128), _cdiv(K, 128))
    for t, name in ((s_in, "s_in"), (s_out, "s_out")):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shape}")
    _check(load_library().fp8q_requant_weight_pow2(_ptr(q_in), ldi, _ptr(s_in), N, K, _ptr(q_out), ldo,
                                                   _ptr(s_out), _stream(stream)), "fp8q_requant_weight_pow2")


def fp8q_quant_weight_block(w, block_n, block_k, fmt, q, scale_inv, stream=None):
    N, K, ldw = _rows(w, torch.bfloat16, "w")
    q = _u8(q)
    _, _, ldq = _rows(q, torch.uint8, "q")
    _check(load_library().fp8q_quant_weight_block(_ptr(w), N, K, ldw, block_n, block_k, fmt,
                                                  _ptr(q), ldq, _ptr(scale_inv), _stream(stream)),
           "fp8q_quant_weight_block")


def fp8q_gemm_blockscale(a, a_scales, a_layout, w, w_scale_inv, bias, y, gran, stream=None):
    a, w = _u8(a), _u8(w)
    M, K, lda = _rows(a, torch.uint8, "a")
    N, Kw, ldw = _rows(w, torch.uint8, "w")
    My, Ny, ldy = _rows(y, torch.bfloat16, "y")
    if Kw != K or (My, Ny) != (M, N):
        raise ValueError("shape mismatch between a, w and y")
    _check(load_library().fp8q_gemm_blockscale(_ptr(a), lda, _ptr(a_scales), a_layout, _ptr(w), ldw,
                                               _ptr(w_scale_inv), _ptr(bias), _ptr(y), ldy, M, N, K,
                                               gran, _stream(stream)), "fp8q_gemm_blockscale")


def fp8q_gemm_splitk_workspace_size(M: int, N: int, K: int) -> int:
    return int(load_library().fp8q_gemm_splitk_workspace_size(M, N, K))


def fp8q_gemm_blockscale_splitk(a, a_scales, a_layout, w, w_scale_inv, bias, y, gran, workspace, stream=None):
    """fp8q_gemm_blockscale with K split over idle CUs; workspace: a device
    tensor (its whole size is offered) or None."""
    a, w = _u8(a), _u8(w)
    M, K, lda = _rows(a, torch.uint8, "a")
    N, Kw, ldw = _rows(w, torch.uint8, "w")
    My, Ny, ldy = _rows(y, torch.bfloat16, "y")
    if Kw != K or (My, Ny) != (M, N):
        raise ValueError("shape mismatch")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().fp8q_gemm_blockscale_splitk(_ptr(a), lda, _ptr(a_scales), a_layout, _ptr(w), ldw,
                                                      _ptr(w_scale_inv), _ptr(bias), _ptr(y), ldy, M, N, K, gran,
                                                      _ptr(workspace), ws_bytes, _stream(stream)),
           "fp8q_gemm_blockscale_splitk")


def fp8q_gemm_blockscale_splitk_noalloc(a, a_scales, a_layout, w, w_scale_inv, bias, y, gran, stream=None):
    """fp8q_gemm_blockscale_splitk with the library's own device scratch
    (no workspace, nothing allocated)."""
    a, w = _u8(a), _u8(w)
    M, K, lda = _rows(a, torch.uint8, "a")
    N, Kw, ldw = _rows(w, torch.uint8, "w")
    My, Ny, ldy = _rows(y, torch.bfloat16, "y")
    if Kw != K or (My, Ny) != (M, N):
        raise ValueError("shape mismatch")
    _check(load_library().fp8q_gemm_blockscale_splitk_noalloc(_ptr(a), lda, _ptr(a_scales), a_layout, _ptr(w),
                                                              ldw, _ptr(w_scale_inv), _ptr(bias), _ptr(y), ldy, M,
                                                              N, K, gran, _stream(stream)),
           "fp8q_gemm_blockscale_splitk_noalloc")


def fp8q_gemm_grouped_blockscale(a, a_scales, a_layout, expert_offsets, w, w_scale_inv, y, shard=0,
                                 gran=GRAN_BLOCK128, stream=None):
    """a [M, K] expert-sorted rows; expert_offsets int32 [E+1] (device);
    w [E, N, K] (uint8 / float8 view, rows 16-byte aligned); w_scale_inv fp32
    [E, NBs, ceil(K/128)]; y bf16 [M, N]."""
    a, w = _u8(a), _u8(w)
    M, K, lda = _rows(a, torch.uint8, "a")
    if w.dim() != 3 or w.stride(2) != 1 or w.size(2) != K:
        raise ValueError("w must be [E, N, K] with unit column stride")
    E, N = w.size(0), w.size(1)
    ldw, w_stride = w.stride(1), w.stride(0)
    My, Ny, ldy = _rows(y, torch.bfloat16, "y")
    if (My, Ny) != (M, N):
        raise ValueError("y must be [M, N]")
    if expert_offsets.dtype != torch.int32 or expert_offsets.numel() != E + 1 or not expert_offsets.is_cuda:
        raise ValueError("expert_offsets must be a device int32 tensor of E + 1 entries")
    if w_scale_inv.dtype != torch.float32 or not w_scale_inv.is_contiguous() or w_scale_inv.size(0) != E:
        raise ValueError("w_scale_inv must be a contiguous float32 [E, NBs, ceil(K/128)] tensor")
    _check(load_library().fp8q_gemm_grouped_blockscale(_ptr(a), lda, _ptr(a_scales), a_layout, _ptr(expert_offsets),
                                                       E, _ptr(w), ldw, w_stride, _ptr(w_scale_inv), shard, _ptr(y),
                                                       ldy, M, N, K, gran, _stream(stream)),
           "fp8q_gemm_grouped_blockscale")


def fp8q_gemm_mxfp8(a, a_scales, w, w_scales, bias, y, scale_layout=ROW_MAJOR, stream=None):
    a, w = _u8(a), _u8(w)
    M, K, lda = _rows(a, torch.uint8, "a")
    N, Kw, ldw = _rows(w, torch.uint8, "w")
    My, Ny, ldy = _rows(y, torch.bfloat16, "y")
    if Kw != K or (My, Ny) != (M, N):
        raise ValueError("shape mismatch between a, w and y")
    _check(load_library().fp8q_gemm_mxfp8(_ptr(a), lda, _ptr(a_scales), _ptr(w), ldw, _ptr(w_scales),
                                          scale_layout, _ptr(bias), _ptr(y), ldy, M, N, K, _stream(stream)),
           "fp8q_gemm_mxfp8")


# --------------------------------------------------------------------------
# allocating helpers


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _q_like(M: int, K: int, device) -> torch.Tensor:
    """uint8 [M, K] view of an [M, ld] buffer with ld a multiple of 16."""
    ld = _cdiv(K, 16) * 16
    return torch.empty(M, ld, dtype=torch.uint8, device=device)[:, :K]


def quant_act_group(x: torch.Tensor, layout: int = ROW_MAJOR, stream=None):
    """(q uint8 [M,K], scales fp32 [M, ceil(K/128)] or [ceil(K/128), M])."""
    M, K = x.shape
    G = _cdiv(K, 128)
    q = _q_like(M, K, x.device)
    s = torch.empty((G, M) if layout == COL_MAJOR else (M, G), dtype=torch.float32, device=x.device)
    fp8q_quant_act_group(x, 128, SCALE_F32, layout, None, q, s, stream)
    return q, s


def quant_act_group_pow2(x: torch.Tensor, layout: int = ROW_MAJOR, stream=None):
    """(q, power-of-two fp32 scales) with 128-wide groups (block FP8 as an MXFP8 view)."""
    M, K = x.shape
    G = _cdiv(K, 128)
    q = _q_like(M, K, x.device)
    s = torch.empty((G, M) if layout == COL_MAJOR else (M, G), dtype=torch.float32, device=x.device)
    fp8q_quant_act_group(x, 128, SCALE_F32_POW2, layout, None, q, s, stream)
    return q, s


def quant_act_mx(x: torch.Tensor, layout: int = ROW_MAJOR, stream=None):
    """(q uint8 [M,K], UE8M0 scale bytes uint8 [M, ceil(K/32)] or [ceil(K/32), M]).
    Also the MX quantizer of weight rows (any layout)."""
    M, K = x.shape
    q = _q_like(M, K, x.device)
    G = _cdiv(K, 32)
    s = torch.empty((G, M) if layout == COL_MAJOR else (M, G), dtype=torch.uint8, device=x.device)
    fp8q_quant_act_group(x, 32, SCALE_UE8M0, layout, None, q, s, stream)
    return q, s


def quant_act_static(x: torch.Tensor, scale: torch.Tensor, stream=None):
    """q uint8 [M,K] with a given device fp32 scalar scale."""
    M, K = x.shape
    q = _q_like(M, K, x.device)
    fp8q_quant_act_group(x, 128, SCALE_F32, ROW_MAJOR, scale, q, None, stream)
    return q


def rmsnorm_quant(x, gamma, eps: float = 1e-6, layout: int = ROW_MAJOR, return_y: bool = False, stream=None):
    """(q, scales[, y]) of RMSNorm(x) followed by group-128 quantization."""
    M, K = x.shape
    G = _cdiv(K, 128)
    q = _q_like(M, K, x.device)
    s = torch.empty((G, M) if layout == COL_MAJOR else (M, G), dtype=torch.float32, device=x.device)
    y = torch.empty(M, K, dtype=torch.bfloat16, device=x.device) if return_y else None
    fp8q_rmsnorm_quant(x, gamma, eps, layout, q, s, y, stream)
    return (q, s, y) if return_y else (q, s)


def add_rmsnorm_quant(x, h, gamma, eps: float = 1e-6, layout: int = ROW_MAJOR, static_scale=None,
                      return_y: bool = False, fmt: int = SCALE_F32, stream=None):
    """Residual add in place (x <- bf16(x + h)), then RMSNorm and quantization.

    Returns (q, scales[, y]); scales is None with a static scale.
    """
    M, K = x.shape
    G = _cdiv(K, 128)
    q = _q_like(M, K, x.device)
    s = None
    if static_scale is None:
        s = torch.empty((G, M) if layout == COL_MAJOR else (M, G), dtype=torch.float32, device=x.device)
    y = torch.empty(M, K, dtype=torch.bfloat16, device=x.device) if return_y else None
    fp8q_add_rmsnorm_quant(x, h, x if h is not None else None, gamma, eps, fmt, layout, static_scale, q, s, y,
                           stream)
    return (q, s, y) if return_y else (q, s)


def rmsnorm_quant_pow2(x, gamma, eps: float = 1e-6, layout: int = ROW_MAJOR, return_y: bool = False,
                       stream=None):
    """(q, power-of-two scales[, y]) of RMSNorm(x) followed by group-128 quantization."""
    return add_rmsnorm_quant(x, None, gamma, eps, layout, None, return_y, SCALE_F32_POW2, stream)


def quant_weight_block(w: torch.Tensor, stream=None):
    """(q uint8 [N,K], scale_inv fp32 [ceil(N/128), ceil(K/128)])."""
    N, K = w.shape
    q = _q_like(N, K, w.device)
    s = torch.empty(_cdiv(N, 128), _cdiv(K, 128), dtype=torch.float32, device=w.device)
    fp8q_quant_weight_block(w, 128, 128, SCALE_F32, q, s, stream)
    return q, s


def quant_weight_block_pow2(w: torch.Tensor, stream=None):
    """(q uint8 [N,K], power-of-two scale_inv fp32 [ceil(N/128), ceil(K/128)])."""
    N, K = w.shape
    q = _q_like(N, K, w.device)
    s = torch.empty(_cdiv(N, 128), _cdiv(K, 128), dtype=torch.float32, device=w.device)
    fp8q_quant_weight_block(w, 128, 128, SCALE_F32_POW2, q, s, stream)
    return q, s


def requant_weight_pow2(q: torch.Tensor, s: torch.Tensor, stream=None):
    """Block-FP8 (q, fp32 block scales) -> (q', power-of-two scales), new buffers."""
    N, K = q.shape
    q2 = _q_like(N, K, q.device)
    s2 = torch.empty_like(s)
    fp8q_requant_weight_pow2(q, s, q2, s2, stream)
    return q2, s2


def quant_weight_mx(w: torch.Tensor, stream=None):
    N, K = w.shape
    q = _q_like(N, K, w.device)
    s = torch.empty(N, _cdiv(K, 32), dtype=torch.uint8, device=w.device)
    fp8q_quant_weight_block(w, 1, 32, SCALE_UE8M0, q, s, stream)
    return q, s


def quant_weight_tensor(w: torch.Tensor, stream=None):
    N, K = w.shape
    q = _q_like(N, K, w.device)
    s = torch.empty(1, dtype=torch.float32, device=w.device)
    fp8q_quant_weight_block(w, N, K, SCALE_F32, q, s, stream)
    return q, s


def _y(M: int, N: int, device) -> torch.Tensor:
    ld = _cdiv(N, 8) * 8
    return torch.empty(M, ld, dtype=torch.bfloat16, device=device)[:, :N]


def gemm_blockscale(a, a_scales, w, w_scale_inv, bias=None, a_layout: int = ROW_MAJOR, stream=None):
    y = _y(a.shape[0], w.shape[0], a.device)
    fp8q_gemm_blockscale(a, a_scales, a_layout, w, w_scale_inv, bias, y, GRAN_BLOCK128, stream)
    return y


def gemm_blockscale_pow2(a, a_scales, w, w_scale_inv, bias=None, a_layout: int = ROW_MAJOR, stream=None):
    """Block GEMM on power-of-two scales, applied by the scaled MFMA."""
    y = _y(a.shape[0], w.shape[0], a.device)
    fp8q_gemm_blockscale(a, a_scales, a_layout, w, w_scale_inv, bias, y, GRAN_BLOCK128_POW2, stream)
    return y


def gemm_blockscale_splitk(a, a_scales, w, w_scale_inv, bias=None, a_layout: int = ROW_MAJOR, gran=GRAN_BLOCK128,
                           workspace=None, stream=None):
    """Block GEMM through the split-K entry (decode shapes split K; prefill
    shapes split their leftover tiles along K); allocates the workspace
    (torch) when none is given."""
    M, N, K = a.shape[0], w.shape[0], a.shape[1]
    if workspace is None:
        nbytes = fp8q_gemm_splitk_workspace_size(M, N, K)
        workspace = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device=a.device) if nbytes else None
    y = _y(M, N, a.device)
    fp8q_gemm_blockscale_splitk(a, a_scales, a_layout, w, w_scale_inv, bias, y, gran, workspace, stream)
    return y


def gemm_grouped_blockscale(a, a_scales, expert_offsets, w, w_scale_inv, shard=0, a_layout: int = ROW_MAJOR,
                            gran=GRAN_BLOCK128, stream=None):
    """MoE expert GEMMs over expert-sorted rows; returns y bf16 [M, N]."""
    y = _y(a.shape[0], w.shape[1], a.device)
    fp8q_gemm_grouped_blockscale(a, a_scales, a_layout, expert_offsets, w, w_scale_inv, y, shard, gran, stream)
    return y


def gemm_pertensor(a, a_scale, w, w_scale, bias=None, stream=None):
    y = _y(a.shape[0], w.shape[0], a.device)
    fp8q_gemm_blockscale(a, a_scale, ROW_MAJOR, w, w_scale, bias, y, GRAN_PER_TENSOR, stream)
    return y


def gemm_mxfp8(a, a_scales, w, w_scales, bias=None, scale_layout=ROW_MAJOR, stream=None):
    y = _y(a.shape[0], w.shape[0], a.device)
    fp8q_gemm_mxfp8(a, a_scales, w, w_scales, bias, y, scale_layout, stream)
    return y
