"""Scaled FP8 GEMMs of the blockwise linear layer (CPU oracle).

Test infrastructure: see the package docstring.

All three compute Y = X W^T for E4M3 codes X [M, K] (activations) and
W [N, K] (weights, row-major [out, in]) and return bf16 Y [M, N].

Definitions followed
--------------------
* Block-wise: Y_ij = sum_b (sum_{k in block b} QX[i,k] QW[j,k]) * s_x[i,b]
  * s_w[j // 128, b]; the scales depend on b so they cannot leave the sum;
  accumulation is fp32 or better, there is no dequantized copy of the weight,
  and the epilogue adds the bias and converts to bf16
  ([SGL19] "一条 GEMM 的三种缩放组合", "Triton 分块内核在做什么",
  "一次前向的完整时序").  ``weight_scale_inv`` is the multiplier s_w, as the
  pages use it.
* Per-tensor: Y = (QX QW^T) * s_x * s_w with scalar scales
  ([SGL19] "一条 GEMM 的三种缩放组合").
* Grouped (MoE experts): the activation rows are sorted by expert and
  contiguous; rows offsets[e] .. offsets[e+1] are multiplied by expert e's
  weight and scales ([SGL19] "MoE:专家权重多一个维度": w13 [E, 2 I_p, H],
  w2 [E, H, I_p], one scale grid per expert; grouped GEMMs take the
  expert-sorted contiguous layout).  With stacked shards (w13's gate and
  up), the weight scale row of output channel j is
  (j // shard) * ceil(shard/128) + (j % shard) // 128.
* MXFP8: the same block identity with 1x32 blocks whose scales are powers of
  two 2^(byte-127) ([SGLFP8] "4. 블록 양자화 스케일 관리"; [SGL19]
  "Triton 分块内核在做什么": UE8M0 scales turn the multiply into an exponent
  add).

Arithmetic: decoded E4M3 values are fp64; every product of two E4M3 values is
a multiple of 2^-18 below 2^18, so any partial sum over up to 2^13 products
is an exactly representable fp64 number -- a BLAS dgemm of decoded values is
exact whatever its summation order.  The scaled block sums are added in fp64
and the result is rounded once to bf16 (RNE).  Block sums are computed
``rows`` at a time to bound memory.
"""
from __future__ import annotations

import numpy as np

from . import bf16, e4m3


def _kb(K: int, bk: int) -> int:
    return -(-K // bk)


def _finish(acc, bias):
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float64)[None, :]
    return bf16.round_from_f64(acc), acc


def weight_scale_rows(N: int, shard: int = 0, block: int = 128) -> np.ndarray:
    """Scale-row index of each output channel j: j // 128, or with stacked
    shards (j // shard) * ceil(shard/128) + (j % shard) // 128."""
    j = np.arange(N)
    if not shard:
        return j // block
    return (j // shard) * (-(-shard // block)) + (j % shard) // block


def gemm_blockscale(qa, sa, qw, sw, bias=None, block: int = 128, rows=None, shard: int = 0):
    """Block-scaled GEMM.  qa uint8 [M,K], sa fp32 [M, ceil(K/128)],
    qw uint8 [N,K], sw fp32 [ceil(N/128), ceil(K/128)] (stacked shards:
    [(N/shard) * ceil(shard/128), ceil(K/128)]), bias fp64-able [N].

    ``rows`` optionally restricts the computation to those output rows.
    Returns (Y bf16 bits [m, N], Y before rounding fp64 [m, N]).
    """
    qa = np.asarray(qa, dtype=np.uint8)
    sa = np.asarray(sa, dtype=np.float32)
    if rows is not None:
        qa, sa = qa[rows], sa[rows]
    A = e4m3.decode(qa)
    W = e4m3.decode(qw)
    M, K = A.shape
    N = W.shape[0]
    sw = np.asarray(sw, dtype=np.float64)
    sw_cols = sw[weight_scale_rows(N, shard, block)]   # [N, KB]: scale of column j's block
    acc = np.zeros((M, N), dtype=np.float64)
    for b in range(_kb(K, block)):
        ks = slice(b * block, min(K, (b + 1) * block))
        P = A[:, ks] @ W[:, ks].T                # exact block sum
        acc += P * sa[:, b].astype(np.float64)[:, None] * sw_cols[:, b][None, :]
    return _finish(acc, bias)


def gemm_grouped_blockscale(qa, sa, qw, sw, offsets, shard: int = 0, rows=None):
    """Grouped block-scaled GEMM over expert-sorted rows.

    qa uint8 [M, K], sa fp32 [M, ceil(K/128)]; qw uint8 [E, N, K] (or a
    callable e -> qw[e]), sw fp32 [E, NBs, ceil(K/128)] (or a callable);
    offsets int [E+1], non-decreasing, offsets[0] = 0, offsets[E] = M.
    ``rows`` restricts the computation to those output rows.
    Returns Y bf16 bits [m, N].
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    M = offsets[-1]
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    get_w = qw if callable(qw) else (lambda e: qw[e])
    get_s = sw if callable(sw) else (lambda e: sw[e])
    expert = np.searchsorted(offsets, rows, side="right") - 1     # expert of each row
    out = None
    for e in np.unique(expert):
        sel = np.flatnonzero(expert == e)
        y, _ = gemm_blockscale(qa, sa, get_w(e), get_s(e), rows=rows[sel], shard=shard)
        if out is None:
            out = np.empty((len(rows), y.shape[1]), dtype=np.uint16)
        out[sel] = y
    if out is None:
        out = np.empty((0, np.asarray(get_w(0)).shape[0]), dtype=np.uint16)
    return out


def gemm_pertensor(qa, sa, qw, sw, bias=None, rows=None):
    """Per-tensor scaled GEMM: scalar sa, sw."""
    qa = np.asarray(qa, dtype=np.uint8)
    if rows is not None:
        qa = qa[rows]
    A = e4m3.decode(qa)
    W = e4m3.decode(qw)
    acc = (A @ W.T) * float(np.float32(sa)) * float(np.float32(sw))
    return _finish(acc, bias)


def gemm_mx(qa, ea, qw, ew, bias=None, block: int = 32, rows=None):
    """MXFP8 GEMM.  ea uint8 [M, ceil(K/32)], ew uint8 [N, ceil(K/32)]."""
    qa = np.asarray(qa, dtype=np.uint8)
    ea = np.asarray(ea, dtype=np.uint8)
    if rows is not None:
        qa, ea = qa[rows], ea[rows]
    A = e4m3.decode(qa)
    W = e4m3.decode(qw)
    M, K = A.shape
    N = W.shape[0]
    xa = ea.astype(np.int64) - 127
    xw = np.asarray(ew, dtype=np.uint8).astype(np.int64) - 127
    acc = np.zeros((M, N), dtype=np.float64)
    for b in range(_kb(K, block)):
        ks = slice(b * block, min(K, (b + 1) * block))
        P = A[:, ks] @ W[:, ks].T
        acc += np.ldexp(P, xa[:, b][:, None] + xw[:, b][None, :])
    return _finish(acc, bias)


# ---------------------------------------------------------------------------
# Second formulations, used only to pin the ones above: dequantize each
# operand to fp64 first (x_hat = q * s, [SGL19] "从浮点到 FP8 的基本公式")
# and run one plain fp64 matmul.


def dequant_groups(q, s, group_rows: int, group_cols: int) -> np.ndarray:
    """q * s with s expanded over group_rows x group_cols blocks (fp64)."""
    v = e4m3.decode(q)
    s = np.asarray(s, dtype=np.float64)
    S = np.repeat(np.repeat(s, group_rows, axis=0), group_cols, axis=1)
    return v * S[: v.shape[0], : v.shape[1]]


def gemm_dequant_reference(qa, sa, qw, sw, block: int = 128) -> np.ndarray:
    """(QX * s_x)(QW * s_w)^T in fp64, unrounded."""
    Xd = dequant_groups(qa, sa, 1, block)
    Wd = dequant_groups(qw, sw, block, block)
    return Xd @ Wd.T


def gemm_mx_dequant_reference(qa, ea, qw, ew, block: int = 32) -> np.ndarray:
    sa = np.ldexp(1.0, np.asarray(ea, np.int64) - 127)
    sw = np.ldexp(1.0, np.asarray(ew, np.int64) - 127)
    return dequant_groups(qa, sa, 1, block) @ dequant_groups(qw, sw, 1, block).T
