"""Quantizers of the FP8 blockwise linear layer (CPU oracle).

Test infrastructure: see the package docstring.

Inputs are bf16 values given as fp32 (or fp64) arrays holding exactly the bf16
values.  Outputs are uint8 E4M3 codes plus scales.

Definitions followed
--------------------
* Quantize / dequantize: q = clamp(round(x/s), -448, 448), x_hat = q*s,
  round = round-to-nearest-even; the clamp keeps outliers from becoming NaN
  ([SGL19] "从浮点到 FP8 的基本公式").
* Dynamic per-token-group activation scale: each run of 128 consecutive
  channels of a row gets s_g = max|x| / 448 and q = round(x / s_g); the
  scales form an [M, ceil(K/128)] fp32 grid, row-major by default
  ([GLM17] "第 1 站:RMSNorm 的两个出口"; [SGL19] "Triton 分块内核在做什么").
* Per-tensor scale s = max|W| / 448 ([SGL19] "从浮点到 FP8 的基本公式").
* Block-wise weight scale: the same rule restricted to each b_n x b_k
  sub-matrix (128x128), on a ceil(N/b_n) x ceil(K/b_k) grid whose last
  row/column of blocks may be partial ([SGL19] "建权重:先决定 scale 的形状",
  "从浮点到 FP8 的基本公式").
* MXFP8: 1x32 blocks, one UE8M0 (power-of-two, uint8) scale each
  ([SGLFP8] "1. Fp8Config 초기화", "4. 블록 양자화 스케일 관리"); the scale
  exponent is rounded UP so the block never overflows:
  scale = 2^ceil(log2(max(amax, 1e-10) / 448))
  ([GLM17] "第 4 站:索引器——FP8 与排名稳定性").
* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, statistics in high precision,
  bf16 output ([GLM17] "第 1 站:RMSNorm 的两个出口").
* Residual add: each decoder layer first adds the sublayer output back into
  the bf16 residual stream and normalizes the sum; with a static per-tensor
  activation scale add, norm and the fixed-scale cast are one step, with
  blockwise weights the group quantizer follows the norm
  ([GLM17] "第 1 站:RMSNorm 的两个出口"; the stream stays bf16 across layers,
  "第 6 站:o_proj、残差流与 AllReduce 为什么停在 BF16").

Readings where the pages leave a step open
------------------------------------------
(i)   x/s is one IEEE fp32 division, then one RNE rounding to E4M3 (the scale
      is fp32, and the kernel computes in fp32).
(ii)  s = amax/448 is an fp32 division, not a multiply by 1/448.
(iii) amax is floored at fp32(1e-10) before dividing (the only floor the pages
      print, in the UE8M0 rule); a zero group gets s = fp32(1e-10)/448, q = 0.
(iv)  clamp to +-448 before the cast.
(v)   the sign of zero is kept (-0 and negatives rounding to zero -> 0x80).
(vi)  RMSNorm: r = 1/sqrt(sum(x^2)/K + eps) is evaluated in fp64 from an
      exactly rounded sum and rounded once to fp32; y = bf16(fp32(fp32(x*r)*g)).
      The quantizer consumes the bf16 y.
(vii) MX exponent: e = the smallest integer with max(amax, 1e-10) <= 448*2^e,
      stored as the byte e + 127; q = E4M3(x * 2^-e) (exact scaling).
(ix)  Power-of-two ("UE8M0") block scales held in fp32: the block-FP8 data
      consumed as an MXFP8 view keeps the 128-wide activation groups and the
      128x128 weight blocks but restricts every scale to a power of two,
      s = 2^e with e from the round-up rule of (vii); q = E4M3(x * 2^-e).
      The fp32 value 2^e carries the UE8M0 byte e + 127 as its exponent field.
(x)   Re-quantizing an existing block (codes q, fp32 scale s) to a power of
      two: e' = the smallest integer with s <= 2^e' (the round-up rule applied
      to s, which stands for amax/448), q' = E4M3(decode(q) * s * 2^-e'); as
      s * 2^-e' <= 1, no code grows past 448.
(xi)  Stacked shards (MoE w13 = [gate; up]): each shard of the output rows
      gets its own ceil grid of 128x128 blocks and the scale rows are
      concatenated, 2 * ceil(I_p/128) rows rather than ceil(2 I_p/128)
      ([SGL19] "MoE:专家权重多一个维度").
(viii) Residual add: the updated stream is z = bf16(x + h), the correctly
      rounded sum (one rounding); RMSNorm and the quantizer then read that
      bf16 z, as they would read it back from memory in the unfused sequence.
      The static exit applies the same formula as the static quantizer,
      q = E4M3(clamp(RN32(y / s))).
"""
from __future__ import annotations

import math

import numpy as np

from . import bf16, e4m3

FP8_MAX = np.float32(448.0)
AMAX_FLOOR = np.float32(1e-10)
UE8M0_BIAS = 127


def _ngroups(K: int, g: int) -> int:
    return -(-K // g)


def group_scale(amax) -> np.ndarray:
    """fp32 scale from a group's max |x|: max(amax, 1e-10) / 448 in fp32."""
    a = np.maximum(np.asarray(amax, dtype=np.float32), AMAX_FLOOR)
    return (a / FP8_MAX).astype(np.float32)          # IEEE fp32 division


def quantize_with_scale(x, s) -> np.ndarray:
    """E4M3 codes of clamp(RN32(x / s), -448, 448); x, s broadcastable fp32."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    t = (x / s).astype(np.float32)                    # IEEE fp32 division
    t = np.clip(t, -FP8_MAX, FP8_MAX)
    return e4m3.encode(t)


def quant_group(x, group: int = 128):
    """Dynamic per-token-group quantization with fp32 scales.

    x: [M, K] bf16 values (fp32 array).  Returns (q uint8 [M, K],
    s float32 [M, ceil(K/group)]) with s in row-major order.
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    G = _ngroups(K, group)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, G), dtype=np.float32)
    for g in range(G):
        cols = slice(g * group, min(K, (g + 1) * group))
        xs = x[:, cols]
        amax = np.max(np.abs(xs), axis=1)
        sg = group_scale(amax)
        s[:, g] = sg
        q[:, cols] = quantize_with_scale(xs, sg[:, None])
    return q, s


def quant_static(x, scale):
    """Static per-tensor activation quantization with a given fp32 scalar."""
    x = np.asarray(x, dtype=np.float32)
    return quantize_with_scale(x, np.float32(scale))


def mx_exponent(amax) -> np.ndarray:
    """Smallest integer e with max(amax, 1e-10) <= 448 * 2^e (reading vii)."""
    a = np.maximum(np.asarray(amax, dtype=np.float32), AMAX_FLOOR).astype(np.float64)
    e = np.ceil(np.log2(a / 448.0)).astype(np.int64)      # estimate ...
    # ... then settled by exact comparisons (448 * 2^e is exact in fp64)
    e = np.where(a <= np.ldexp(448.0, e - 1), e - 1, e)
    e = np.where(a > np.ldexp(448.0, e), e + 1, e)
    return e


def quant_mx(x, group: int = 32):
    """MXFP8: 1 x group blocks with UE8M0 scale bytes.

    Returns (q uint8 [M, K], scale bytes uint8 [M, ceil(K/group)]).
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    G = _ngroups(K, group)
    q = np.empty((M, K), dtype=np.uint8)
    sb = np.empty((M, G), dtype=np.uint8)
    for g in range(G):
        cols = slice(g * group, min(K, (g + 1) * group))
        xs = x[:, cols].astype(np.float64)
        e = mx_exponent(np.max(np.abs(xs), axis=1))
        sb[:, g] = (e + UE8M0_BIAS).astype(np.uint8)
        t = np.ldexp(xs, -e[:, None])                    # exact power-of-two scaling
        q[:, cols] = e4m3.encode(np.clip(t, -448.0, 448.0))
    return q, sb


def quant_weight_block(w, block_n: int = 128, block_k: int = 128):
    """Block-wise weight quantization: one fp32 scale per block_n x block_k.

    Returns (q uint8 [N, K], s float32 [ceil(N/block_n), ceil(K/block_k)]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    NB, KB = _ngroups(N, block_n), _ngroups(K, block_k)
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((NB, KB), dtype=np.float32)
    for i in range(NB):
        rows = slice(i * block_n, min(N, (i + 1) * block_n))
        for j in range(KB):
            cols = slice(j * block_k, min(K, (j + 1) * block_k))
            blk = w[rows, cols]
            sb = group_scale(np.max(np.abs(blk)))
            s[i, j] = sb
            q[rows, cols] = quantize_with_scale(blk, sb)
    return q, s


def quant_tensor(w):
    """Per-tensor quantization: one fp32 scale for the whole matrix."""
    w = np.asarray(w, dtype=np.float32)
    s = group_scale(np.max(np.abs(w)))
    return quantize_with_scale(w, s), np.float32(s)


def rms_inv(x, eps: float):
    """Per-row r = RN32(1/sqrt(sum(x^2)/K + eps)) plus near-tie information.

    The sum of squares of bf16 values is taken exactly rounded (math.fsum of
    exact fp64 squares); mean, +eps, sqrt and reciprocal run in fp64.
    Returns (r float32 [M], r_alt float32 [M], ambiguous bool [M]): a row is
    ambiguous when its fp64 value lies within 2^-40 (relative) of the midpoint
    between two fp32 numbers -- there any fp64 evaluation order may round to
    either neighbour, and r_alt is the other one.
    """
    x64 = np.asarray(x, dtype=np.float64)
    M, K = x64.shape
    ss = np.array([math.fsum(row) for row in (x64 * x64)], dtype=np.float64)
    r64 = 1.0 / np.sqrt(ss / K + float(np.float32(eps)))
    r = r64.astype(np.float32)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(0))
    other = np.where(r64 >= r.astype(np.float64), up, dn).astype(np.float32)
    mid = (r.astype(np.float64) + other.astype(np.float64)) * 0.5
    ambiguous = np.abs(r64 - mid) <= np.abs(r64) * 2.0 ** -40
    return r, other, ambiguous


def rmsnorm_apply(x, g, r):
    """y = bf16(fp32(fp32(x * r) * g)) for given per-row fp32 r; uint16 bits."""
    x32 = np.asarray(x, dtype=np.float32)
    g32 = np.asarray(g, dtype=np.float32)
    t = (x32 * np.asarray(r, dtype=np.float32)[:, None]).astype(np.float32)
    t = (t * g32[None, :]).astype(np.float32)
    return bf16.round_from_f64(t.astype(np.float64))


def rmsnorm(x, g, eps: float):
    """RMSNorm with bf16 output.  Returns (y bits uint16 [M,K], r, r_alt, ambiguous)."""
    r, r_alt, amb = rms_inv(x, eps)
    return rmsnorm_apply(x, g, r), r, r_alt, amb


def rmsnorm_quant(x, g, eps: float, group: int = 128, r=None):
    """RMSNorm -> bf16 -> dynamic group quantization (reading vi).

    Returns dict(q, s, y, r, r_alt, ambiguous).  Pass ``r`` to evaluate the
    same pipeline with a chosen per-row factor (used for near-tie rows).
    """
    if r is None:
        r, r_alt, amb = rms_inv(x, eps)
    else:
        r_alt, amb = None, None
    y = rmsnorm_apply(x, g, r)
    q, s = quant_group(bf16.to_f32(y), group)
    return {"q": q, "s": s, "y": y, "r": r, "r_alt": r_alt, "ambiguous": amb}


def residual_add(x, h):
    """Updated residual stream z = bf16(x + h), correctly rounded (reading viii).

    x and h hold bf16 values.  Their fp64 sum is rounded to bf16 once: an
    fp64 sum of two 8-bit-significand values rounded again to 8 bits gives the
    correctly rounded result, because 53 >= 2*8 + 1 (the classical condition
    under which a double rounding through the wider format is innocuous for
    addition).  Returns uint16 bits.
    """
    return bf16.round_from_f64(np.asarray(x, dtype=np.float64) + np.asarray(h, dtype=np.float64))


def add_rmsnorm_quant(x, h, g, eps: float, static_scale=None, group: int = 128, r=None, pow2: bool = False):
    """Residual add -> RMSNorm -> bf16 -> quantization (readings vi, viii, ix).

    static_scale None: dynamic group quantization (q, s per group; power-of-two
    scales if pow2); otherwise per-tensor static quantization with that fp32
    scale (s = None).
    Returns dict(z, q, s, y, r, r_alt, ambiguous); pass ``r`` to evaluate the
    pipeline with a chosen per-row factor (for near-tie rows).
    """
    z = residual_add(x, h)
    zf = bf16.to_f32(z)
    if r is None:
        r, r_alt, amb = rms_inv(zf, eps)
    else:
        r_alt, amb = None, None
    y = rmsnorm_apply(zf, g, r)
    if static_scale is not None:
        q, s = quant_static(bf16.to_f32(y), static_scale), None
    elif pow2:
        q, s = quant_group_pow2(bf16.to_f32(y), group)
    else:
        q, s = quant_group(bf16.to_f32(y), group)
    return {"z": z, "q": q, "s": s, "y": y, "r": r, "r_alt": r_alt, "ambiguous": amb}


def pow2_scale(e) -> np.ndarray:
    """fp32 value 2^e of integer exponents (exact)."""
    return np.ldexp(1.0, np.asarray(e, dtype=np.int64)).astype(np.float32)


def quant_group_pow2(x, group: int = 128):
    """Per-token-group quantization with power-of-two fp32 scales (reading ix).

    The group's exponent follows the MX round-up rule, so this is the MX
    quantizer with 128-wide groups and the scale stored as the fp32 2^e.
    Returns (q uint8 [M, K], s float32 [M, ceil(K/group)]).
    """
    q, sb = quant_mx(x, group)
    return q, pow2_scale(sb.astype(np.int64) - UE8M0_BIAS)


def quant_weight_block_pow2(w, block_n: int = 128, block_k: int = 128):
    """128x128 weight blocks with power-of-two fp32 scales (reading ix).

    Returns (q uint8 [N, K], s float32 [ceil(N/128), ceil(K/128)]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    NB, KB = _ngroups(N, block_n), _ngroups(K, block_k)
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((NB, KB), dtype=np.float32)
    for i in range(NB):
        rows = slice(i * block_n, min(N, (i + 1) * block_n))
        for j in range(KB):
            cols = slice(j * block_k, min(K, (j + 1) * block_k))
            blk = w[rows, cols].astype(np.float64)
            e = int(mx_exponent(np.max(np.abs(blk))))
            s[i, j] = pow2_scale(e)
            q[rows, cols] = e4m3.encode(np.clip(np.ldexp(blk, -e), -448.0, 448.0))
    return q, s


def requant_weight_pow2(q, s, block_n: int = 128, block_k: int = 128):
    """Re-quantize block-FP8 weights (codes q, fp32 block scales s) to
    power-of-two block scales (reading x).  Returns (q', s')."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    N, K = q.shape
    f, k = np.frexp(s.astype(np.float64))          # s = f * 2^k, f in [0.5, 1)
    e = np.where(f == 0.5, k - 1, k).astype(np.int64)
    s2 = pow2_scale(e)
    m = s.astype(np.float64) / s2.astype(np.float64)   # exact: in (1/2, 1]
    mult = np.repeat(np.repeat(m, block_n, axis=0), block_k, axis=1)[:N, :K]
    v = e4m3.decode(q) * mult                       # exact in fp64 (4 x 24 bits)
    return e4m3.encode(np.clip(v, -448.0, 448.0)), s2


def quant_weight_block_sharded(w, shard: int):
    """Block quantization of stacked shards of `shard` output rows each
    (reading xi).  Returns (q [N, K], s [(N/shard) * ceil(shard/128), ceil(K/128)])."""
    w = np.asarray(w, dtype=np.float32)
    N = w.shape[0]
    if shard <= 0 or N % shard:
        raise ValueError("N must be a multiple of the shard size")
    parts = [quant_weight_block(w[i:i + shard]) for i in range(0, N, shard)]
    return np.concatenate([q for q, _ in parts]), np.concatenate([s for _, s in parts])
