"""bfloat16 helpers: bit-pattern decode and round-to-nearest-even from fp64.

Test infrastructure: see the package docstring.

bf16 is the activation, weight and output type of the linear layer
([SGL19] "一次前向的完整时序": the epilogue converts back to BF16;
[GLM17] "第 1 站:RMSNorm 的两个出口": residual stream and norm output BF16).
A bf16 value is the upper 16 bits of an fp32 word: 8 significant bits,
exponent range as fp32, subnormals spaced 2^-133.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float((2.0 - 2.0 ** -7) * 2.0 ** 127)


def to_f64(bits) -> np.ndarray:
    """Value of uint16 bf16 bit patterns, as fp64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f32(bits) -> np.ndarray:
    """Value of uint16 bf16 bit patterns, as fp32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def round_from_f64(v) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) in ONE rounding.

    Written from the definition: keep 8 significant bits (quantum
    2^(e-7) for a value in [2^e, 2^(e+1)), but never finer than the subnormal
    spacing 2^-133); values at or beyond the overflow threshold give +-inf.
    Returns uint16 bit patterns.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN input")
    a = np.abs(v)
    _, e2 = np.frexp(a)                  # a = f * 2^e2, f in [0.5, 1)
    e = e2.astype(np.int64) - 1           # a in [2^e, 2^(e+1))
    q_exp = np.maximum(e, -126) - 7       # log2 of the bf16 quantum here
    q_exp = np.where(a == 0, -133, q_exp)
    n = np.ldexp(a, -q_exp)               # exact: power-of-two scaling
    r = np.ldexp(np.rint(n), q_exp)       # np.rint rounds half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    r = np.copysign(r, v)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
