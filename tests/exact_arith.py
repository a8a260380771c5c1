"""Exact reference arithmetic for pinning the oracle (test code, CPU only).

The oracle computes the quotients of the quantize formula with numpy's fp32
division and encodes with a table search.  The functions here reach the same
results by other means, so that a slip in either is visible:

* ``rn32_quotient(x, s)``: the binary32 round-to-nearest-even value of the
  exact rational x / s, from integer significands (an integer division and
  its remainder), for finite fp32 x and positive normal fp32 s.  Subnormal
  and overflowing quotients follow IEEE-754 (quantum 2^-149; results of
  2^128 and beyond become infinite).
* ``e4m3_nearest(t)``: the E4M3 ("fn") code nearest to each |t| <= 448 by
  brute force over all 127 non-negative finite values, ties to the even code,
  sign from the sign bit of t.  The value set is torch's own decode of the
  codes 0x00..0x7E, not the oracle's table.

Nothing here imports the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

_E4M3 = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _split(v32: np.ndarray):
    """|v| = m * 2^e with integer m (fp32 bit fields); v finite."""
    bits = np.asarray(v32, np.float32).view(np.uint32).astype(np.int64)
    ex = (bits >> 23) & 0xFF
    fr = bits & 0x7FFFFF
    m = np.where(ex > 0, fr | 0x800000, fr)
    e = np.where(ex > 0, ex - 150, -149)
    return m, e, (bits >> 31) & 1


def _normalize24(m, e):
    """Shift nonzero integer significands into [2^23, 2^24)."""
    m = m.copy()
    e = e.copy()
    for sh in (16, 8, 4, 2, 1):
        small = (m > 0) & (m < (1 << (24 - sh)))
        m = np.where(small, m << sh, m)
        e = np.where(small, e - sh, e)
    return m, e


def _bitlen(v):
    """Bit length of positive int64 values below 2^62."""
    n = np.zeros(v.shape, np.int64)
    w = v.copy()
    for sh in (32, 16, 8, 4, 2, 1):
        big = w >= (1 << sh)
        w = np.where(big, w >> sh, w)
        n = np.where(big, n + sh, n)
    return n + (w > 0)


def rn32_quotient(x, s) -> np.ndarray:
    """RN32(x / s) as fp64 (exact), x finite fp32, s positive normal fp32."""
    x = np.asarray(x, np.float32)
    s = np.broadcast_to(np.asarray(s, np.float32), x.shape)
    assert np.all(np.isfinite(x)) and np.all(s > 0) and np.all(np.isfinite(s))
    mx, ex, sx = _split(x)
    ms, es, _ = _split(s)
    assert np.all(ms >= (1 << 23)), "s must be normal"
    zero = mx == 0
    mx, ex = _normalize24(np.where(zero, 1 << 23, mx), ex)
    # x / s = (mx << 39) / ms * 2^(ex - es - 39); the integer quotient has
    # 39 or 40 bits, the remainder is the sticky part
    num = mx << 39
    qint = num // ms
    rem = num - qint * ms
    base = ex - es - 39                        # exponent of qint's unit
    top = _bitlen(qint) - 1 + base             # floor(log2(x/s)) (qint has >= 39 bits)
    quantum = np.maximum(top - 23, -149)       # log2 of the fp32 spacing there
    shift = quantum - base                     # low bits of qint to round off (>= 15)
    shift = np.minimum(shift, 61)              # past 41 the kept part is 0 and no tie is possible
    keep = qint >> shift
    low = qint - (keep << shift)
    half = np.int64(1) << (shift - 1)
    up = (low > half) | ((low == half) & ((rem != 0) | ((keep & 1) == 1)))
    keep = keep + up
    val = np.ldexp(keep.astype(np.float64), quantum)   # exact: keep <= 2^24
    val = np.where(val >= 2.0 ** 128, np.inf, val)
    val = np.where(zero, 0.0, val)
    return np.where(sx == 1, -val, val)


def e4m3_nearest(t) -> np.ndarray:
    """Nearest E4M3 code of each t (|t| <= 448), ties to even, sign of t kept."""
    t = np.asarray(t, np.float64)
    a = np.abs(t)
    assert np.all(a <= 448.0)
    out = np.empty(a.shape, np.uint8)
    flat_a, flat_o = a.reshape(-1), out.reshape(-1)
    for i in range(0, flat_a.size, 1 << 15):
        d = np.abs(_E4M3[None, :] - flat_a[i:i + (1 << 15), None])
        dmin = d.min(axis=1, keepdims=True)
        hit = d == dmin
        # at most two adjacent codes tie: prefer the even one
        first = hit.argmax(axis=1)
        two = hit.sum(axis=1) == 2
        code = np.where(two & (first % 2 == 1), first + 1, first)
        flat_o[i:i + (1 << 15)] = code
    return out | (np.signbit(t).astype(np.uint8) << 7)


def quantize_exact(x, s, clamp=448.0) -> np.ndarray:
    """E4M3(clamp(RN32(x / s), +-448)) by the functions above."""
    t = rn32_quotient(x, s)
    return e4m3_nearest(np.clip(t, -clamp, clamp))
