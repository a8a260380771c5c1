"""Seeded synthetic inputs for the FP8 blockwise linear layer.

This module only draws random numbers and stores them in bf16; it holds none
of the quantization or GEMM arithmetic.  Both the CPU oracle (``oracle/``) and
the HIP path (``fp8_block_scaled_token_amd``) consume what it produces, and it
imports neither of them.

Shapes follow the hidden sizes the source pages work with: 6144 (the GLM-5.3
residual stream, page "GLM-5.3 推理全链路(十七):精度账本", section
"先把 GLM-5.3 的数值常量摆出来") and 7168 (the DeepSeek-V3 weight example,
page "SGLang 源码完全拆解(十九)", section "建权重:先决定 scale 的形状").
The pages name no dataset; every tensor here is synthetic.

Recipe (all draws in fp32 from a torch CPU ``Generator``, then rounded to bf16
with round-to-nearest-even):

* activations ~ N(0, 1); when ``outlier_frac`` > 0, ``round(outlier_frac*K)``
  channels (chosen by a seeded permutation) are multiplied by ``outlier_mult``
  in every row;
* weights ~ N(0, std) with std = 1/sqrt(K) unless stated;
* RMSNorm gain g ~ U(0.5, 1.5);
* sublayer output added to the residual stream: activations of their own
  seed (outlier channels included) times 0.25, an exact power-of-two scaling.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "activations",
    "weights",
    "gamma",
    "make_generator",
]


def make_generator(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def activations(M: int, K: int, seed: int, outlier_frac: float = 0.0,
                outlier_mult: float = 50.0, device: str = "cpu") -> torch.Tensor:
    """bf16 [M, K] ~ N(0,1) with optional outlier channels (see module doc)."""
    gen = make_generator(seed, device)
    x = torch.randn(M, K, generator=gen, dtype=torch.float32, device=device)
    n_out = int(round(outlier_frac * K))
    if n_out > 0:
        gen_c = make_generator(seed + 1_000_003, "cpu")
        cols = torch.randperm(K, generator=gen_c)[:n_out].to(device)
        x[:, cols] *= outlier_mult
    return x.to(torch.bfloat16)


def weights(N: int, K: int, seed: int, std: float | None = None,
            device: str = "cpu") -> torch.Tensor:
    """bf16 [N, K] ~ N(0, std), std defaults to 1/sqrt(K)."""
    if std is None:
        std = 1.0 / math.sqrt(K)
    gen = make_generator(seed, device)
    w = torch.randn(N, K, generator=gen, dtype=torch.float32, device=device)
    return (w * std).to(torch.bfloat16)


def gamma(K: int, seed: int, device: str = "cpu") -> torch.Tensor:
    """bf16 [K] ~ U(0.5, 1.5)."""
    gen = make_generator(seed, device)
    g = torch.rand(K, generator=gen, dtype=torch.float32, device=device) + 0.5
    return g.to(torch.bfloat16)


@dataclass(frozen=True)
class Workload:
    """One named synthetic workload of the blockwise linear layer."""
    name: str
    M: int
    N: int
    K: int
    seed: int
    outlier_frac: float = 0.0
    w_std: float | None = None      # None -> 1/sqrt(K)
    norm: bool = False              # RMSNorm front end (eps 1e-6, g ~ U(0.5,1.5))
    residual: bool = False          # residual add before the norm (h = 0.25 x N(0,1) + outliers)
    mx: bool = False                # also exercised with 1x32 UE8M0 scales

    def make(self, device: str = "cpu") -> dict:
        s = self.seed * 10
        d = {
            "x": activations(self.M, self.K, s + 1, self.outlier_frac, device=device),
            "w": weights(self.N, self.K, s + 2, self.w_std, device=device),
        }
        if self.norm:
            d["gamma"] = gamma(self.K, s + 3, device=device)
            d["eps"] = 1e-6
        if self.residual:
            h = activations(self.M, self.K, s + 4, self.outlier_frac, device=device)
            d["h"] = (h.float() * 0.25).to(torch.bfloat16)
        return d


WORKLOADS = {
    # tiny: A [16,512], W [256,512]
    "tiny": Workload("tiny", 16, 256, 512, seed=0),
    # decode-shaped: A [32,6144] with 0.1% outlier channels x50, W [24576,6144]
    "decode": Workload("decode", 32, 24576, 6144, seed=1, outlier_frac=0.001),
    # prefill-shaped with RMSNorm front end: x [4096,6144], W [6144,6144]
    "prefill_norm": Workload("prefill_norm", 4096, 6144, 6144, seed=2,
                             outlier_frac=0.001, norm=True),
    # the same with the residual add in front: z = x + h -> RMSNorm -> quant
    "prefill_addnorm": Workload("prefill_addnorm", 4096, 6144, 6144, seed=2,
                                outlier_frac=0.001, norm=True, residual=True),
    # large prefill: A [8192,7168] with outliers, W [18432,7168]
    "large": Workload("large", 8192, 18432, 7168, seed=3, outlier_frac=0.001),
    # MXFP8 / per-tensor: A [2048,7168], W [7168,7168], both N(0,1)
    "mx": Workload("mx", 2048, 7168, 7168, seed=4, w_std=1.0, mx=True),
}
