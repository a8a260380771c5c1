"""E4M3 ("fn" variant) codec written out from the format definition.

Test infrastructure: see the package docstring.

Format facts used (all stated by the pages):
* 1 sign bit, 4 exponent bits, 3 mantissa bits; largest finite value 448;
  smallest normal about 2^-6 ([GLM17] "先把 GLM-5.3 的数值常量摆出来";
  [SGL19] "建权重:先决定 scale 的形状" -- only e4m3fn is used, max 448).
* The "fn" variant has no infinities; the all-ones exponent with all-ones
  mantissa (codes 0x7F / 0xFF) is NaN, so every other code is finite.
* Quantization rounds to nearest with ties to even ([SGL19]
  "从浮点到 FP8 的基本公式": round is round-to-nearest-even).

The encoder is a search over the table of the 127 non-negative finite values
(codes 0x00..0x7E, which are in ascending order): a magnitude is compared
with the exact midpoint between its two neighbouring table values.  It is
deliberately unlike any arithmetic or hardware conversion.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def decode_code(code: int) -> float:
    """Value of one 8-bit code, from the sign/exponent/mantissa fields."""
    sign = (code >> 7) & 1
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6            # subnormal: 0.mmm * 2^(1-7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)  # normal: 1.mmm * 2^(e-7)
    return -mag if sign else mag


#: value of every code (fp64, exact); index = code
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

#: non-negative finite magnitudes, codes 0x00..0x7E, strictly ascending
_POS = DECODE_TABLE[:127].copy()


def decode(codes) -> np.ndarray:
    """Decode an array of uint8 codes to fp64 values (NaN for 0x7F/0xFF)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(v) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even code.

    ``v`` must be finite with |v| <= 448 (callers clamp first, as the
    quantize formula does).  The sign of ``v`` is kept, so -0.0 and negative
    values that round to zero give 0x80.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if not np.all(np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("encode expects finite inputs with |v| <= 448")
    lo = np.searchsorted(_POS, a, side="right") - 1     # largest value <= a
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    mid = (_POS[lo] + _POS[hi]) * 0.5                  # exact in fp64
    even_of_pair = np.where(lo % 2 == 0, lo, hi)
    code = np.where(a < mid, lo, np.where(a > mid, hi, even_of_pair))
    sign = np.signbit(v).astype(np.int64)
    return (code.astype(np.int64) | (sign << 7)).astype(np.uint8)
