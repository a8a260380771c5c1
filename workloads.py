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
  seed (outlier channels included) times 0.25, an exact power-of-two scaling;
* MoE routing (synthetic, the GEMM's input layout only): every token picks
  top_k distinct experts uniformly at random (the top_k largest of uniform
  draws); the (token, expert) pairs whose expert is local are sorted by
  expert, then token, and the token rows are gathered in that order.  Expert
  weights are drawn per expert from seed + expert, so any expert can be
  regenerated alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "MoeWorkload",
    "MOE_WORKLOADS",
    "moe_routing",
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
    # narrow, long weight at decode batch size (the split-K case): A [32,28672], W [2048,28672]
    "decode_splitk": Workload("decode_splitk", 32, 2048, 28672, seed=5, outlier_frac=0.001),
    # MXFP8 / per-tensor: A [2048,7168], W [7168,7168], both N(0,1)
    "mx": Workload("mx", 2048, 7168, 7168, seed=4, w_std=1.0, mx=True),
}


def moe_routing(tokens: int, top_k: int, n_experts: int, local_experts: int, seed: int):
    """(token index of each dispatched row [M], offsets [local_experts + 1]).

    Rows are sorted by expert, then by token; rows offsets[e] .. offsets[e+1]
    go to local expert e (experts 0 .. local_experts - 1 are local).
    """
    gen = make_generator(seed)
    picks = torch.rand(tokens, n_experts, generator=gen).topk(top_k, dim=1).indices   # [T, top_k]
    tok = torch.arange(tokens).repeat_interleave(top_k)
    exp = picks.reshape(-1)
    keep = exp < local_experts
    tok, exp = tok[keep], exp[keep]
    order = torch.argsort(exp * tokens + tok)
    tok, exp = tok[order], exp[order]
    counts = torch.bincount(exp, minlength=local_experts)
    offsets = torch.zeros(local_experts + 1, dtype=torch.int64)
    offsets[1:] = torch.cumsum(counts, 0)
    return tok, offsets


@dataclass(frozen=True)
class MoeWorkload:
    """Expert GEMMs of one MoE layer on one GPU's share of the experts."""
    name: str
    tokens: int
    top_k: int
    n_experts: int       # routed experts of the layer
    local_experts: int   # experts held by this GPU
    hidden: int          # H
    inter: int           # I_p
    proj: str            # "up" (w13: N = 2 I_p, K = H, gate/up shards) or "down" (w2: N = H, K = I_p)
    seed: int

    @property
    def N(self) -> int:
        return 2 * self.inter if self.proj == "up" else self.hidden

    @property
    def K(self) -> int:
        return self.hidden if self.proj == "up" else self.inter

    @property
    def shard(self) -> int:
        return self.inter if self.proj == "up" else 0

    def routing(self):
        return moe_routing(self.tokens, self.top_k, self.n_experts, self.local_experts, self.seed * 10 + 5)

    def activations(self, device: str = "cpu") -> torch.Tensor:
        """Dispatched (expert-sorted) input rows [M, K]."""
        tok, _ = self.routing()
        x = activations(self.tokens, self.K, self.seed * 10 + 1, 0.001, device="cpu")
        return x[tok].to(device)

    def expert_weight(self, e: int, device: str = "cpu") -> torch.Tensor:
        return weights(self.N, self.K, self.seed * 1000 + e, device=device)


MOE_WORKLOADS = {
    # the pages' example layer (H 7168, I_p 2048, 256 experts, top-8) with
    # experts split over 8 GPUs: 32 local experts, 4096 tokens
    "moe_up": MoeWorkload("moe_up", 4096, 8, 256, 32, 7168, 2048, "up", seed=7),
    "moe_down": MoeWorkload("moe_down", 4096, 8, 256, 32, 7168, 2048, "down", seed=8),
}
