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


def gemm_blockscale(qa, sa, qw, sw, bias=None, block: int = 128, rows=None):
    """Block-scaled GEMM.  qa uint8 [M,K], sa fp32 [M, ceil(K/128)],
    qw uint8 [N,K], sw fp32 [ceil(N/128), ceil(K/128)], bias fp64-able [N].

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
    sw_cols = sw[np.arange(N) // block]          # [N, KB]: scale of column j's block
    acc = np.zeros((M, N), dtype=np.float64)
    for b in range(_kb(K, block)):
        ks = slice(b * block, min(K, (b + 1) * block))
        P = A[:, ks] @ W[:, ks].T                # exact block sum
        acc += P * sa[:, b].astype(np.float64)[:, None] * sw_cols[:, b][None, :]
    return _finish(acc, bias)


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
