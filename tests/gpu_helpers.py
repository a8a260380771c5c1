"""Helpers for the GPU parity tests: padded device buffers with canaries,
host/device conversion, and the GEMM tolerance check.

Inputs come from ``workloads`` (seeded, synthetic) or from small seeded
generators here; expected values come only from ``oracle``.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

CANARY_U8 = 0xA5
CANARY_BF16 = 0x7FC1          # a NaN pattern no kernel writes


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_host(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> fp32 numpy holding the same values."""
    return x.detach().to("cpu").float().numpy()


def padded(rows: int, cols: int, dtype: torch.dtype, pad: int, fill: int):
    """Device buffer [rows, ld] filled with a canary; returns (buffer, view[:, :cols]).

    ld is cols + pad rounded up so that rows start on 16-byte boundaries.
    """
    elem = torch.tensor([], dtype=dtype).element_size()
    per16 = 16 // elem
    ld = -(-(cols + pad) // per16) * per16
    if dtype == torch.bfloat16:
        buf = torch.full((rows, ld), 0, dtype=torch.int16, device="cuda")
        buf.fill_(np.int16(np.uint16(fill).view(np.int16)).item())
        buf = buf.view(torch.bfloat16)
    else:
        buf = torch.full((rows, ld), fill, dtype=dtype, device="cuda")
    return buf, buf[:, :cols]


def canary_intact(buf: torch.Tensor, cols: int, fill: int) -> bool:
    tail = buf[:, cols:]
    if tail.numel() == 0:
        return True
    if tail.dtype == torch.bfloat16:
        return bool((tail.view(torch.int16).to(torch.int32) & 0xFFFF).eq(fill).all().item())
    return bool(tail.eq(fill).all().item())


def bf16_bits(y: torch.Tensor) -> np.ndarray:
    return y.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def check_gemm_rows(y_gpu_bits: np.ndarray, y_ref_bits: np.ndarray, what: str, rel: float = 1e-2):
    """Per row: max |Y_gpu - Y_ref| <= rel * max |Y_ref| (bf16 values)."""
    from oracle import bf16 as obf16
    g = obf16.to_f64(y_gpu_bits)
    r = obf16.to_f64(y_ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r).max(axis=1)
    scale = np.abs(r).max(axis=1)
    worst = float(np.max(err / np.maximum(scale, 1e-300)))
    same = float(np.mean(y_gpu_bits == y_ref_bits))
    log(f"{what}: worst row rel err {worst:.3e}, bit-equal {100 * same:.2f}%")
    assert np.all(err <= rel * scale), f"{what}: tolerance exceeded (worst {worst:.3e})"
    return worst, same
