"""Seeded synthetic inputs for the NVFP4 GEMM workloads.

This module only draws random numbers and builds index bookkeeping (MoE
routing); it holds none of the NVFP4 arithmetic (no quantisation, no
decoding, no GEMM).  Both the CPU oracle side of the tests and the GPU side
take their inputs from here, so the two always see the same values.

Shapes follow the pages:
  * NVFP4 linear layer, in_features = out_features = 8192 (kernelindex,
    "NVFP4 linear layer", workload line: sf_k, in_features, sf_vec_size,
    out_features, in_features_half).  Its M values are not published; the
    linear workload uses M = 4096.
  * Decode-shaped GEMMs with M of 16..64 tokens (magik.net "The Moment of
    Recalibration", section "Input Knowledge", previous benchmark results).
  * MoE with 256 experts, 8 active per token, 512 concurrent requests giving
    ~16 tokens per expert (same page, "MoE architecture implications"); the
    per-expert GEMM shape K=2048, N=6144 ("The Moment of Synthesis", section
    "The Reasoning Process", third point).

Value recipe: fp32 standard normals from a CPU ``torch.Generator`` (or a CUDA
generator for the multi-GB MoE weights), optionally with an independent
Bernoulli(0.01) mask of entries multiplied by 50, then cast to bf16 with
round-to-nearest-even where the workload is bf16.
"""
from __future__ import annotations

import dataclasses

import torch

# ---------------------------------------------------------------------------
# workload table
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_dtype: str      # "fp32" or "bf16": dtype of x and W before quantisation
    out_dtype: str     # "f32" or "bf16"
    outliers: bool = False


TINY = Workload("tiny_m128_n256_k512", 128, 256, 512, "fp32", "f32")
LINEAR = Workload("linear_m4096_n8192_k8192", 4096, 8192, 8192, "bf16", "bf16")
DECODE = {m: Workload(f"decode_m{m}_n8192_k8192", m, 8192, 8192, "bf16", "bf16")
          for m in (1, 16, 32)}
LARGE = Workload("large_m16384_n16384_k16384_outliers", 16384, 16384, 16384,
                 "bf16", "bf16", outliers=True)

MOE_TOKENS = 512
MOE_EXPERTS = 256
MOE_TOPK = 8
MOE_GATE_UP = (4096, 6144)   # (N, K) per expert
MOE_DOWN = (6144, 2048)      # (N, K) per expert


def seed_for(config: int, tensor_index: int) -> int:
    """Seed convention: 1000 * workload index + tensor index."""
    return 1000 * config + tensor_index


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------


def randn(shape, seed: int, dtype: str = "fp32", outliers: bool = False,
          device: str = "cpu") -> torch.Tensor:
    """Seeded N(0,1) tensor, optional 1 % x50 outliers, cast to ``dtype``.

    The draw happens in fp32; the outlier mask is a second, independent draw
    from the same generator; the bf16 cast is torch's round-to-nearest-even.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if outliers:
        mask = torch.rand(*shape, generator=gen, dtype=torch.float32,
                          device=device) < 0.01
        x = torch.where(mask, x * 50.0, x)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp32":
        return x
    raise ValueError(dtype)


def gemm_inputs(config: int, wl: Workload, device: str = "cpu"):
    """x [M, K] drawn before W [N, K] (seeds 1000c+0 and 1000c+1)."""
    x = randn((wl.M, wl.K), seed_for(config, 0), wl.in_dtype, wl.outliers, device)
    w = randn((wl.N, wl.K), seed_for(config, 1), wl.in_dtype, wl.outliers, device)
    return x, w


@dataclasses.dataclass
class MoeRouting:
    expert_of: torch.Tensor      # [tokens, topk] int64, chosen experts
    row_token: torch.Tensor      # [tokens*topk] int64, token of each sorted row
    m_offsets: torch.Tensor      # [experts+1] int32, rows of expert e: [off[e], off[e+1])

    @property
    def counts(self) -> torch.Tensor:
        return self.m_offsets[1:] - self.m_offsets[:-1]


def moe_routing(seed: int, tokens: int = MOE_TOKENS, experts: int = MOE_EXPERTS,
                topk: int = MOE_TOPK, skew: float = 0.0) -> MoeRouting:
    """Seeded softmax router over N(0,1) logits, top-k, rows sorted stably by
    (expert, token).  Routing is harness bookkeeping, not part of the GEMM.
    ``skew`` > 0 lowers expert e's logit by skew * log(1 + e), so a few
    experts draw most tokens and many draw none (the uneven routing expected
    in practice: "The Moment of Synthesis", "Assumptions and Potential
    Mistakes"); skew 1.0 at 512 tokens x top-8 of 256 leaves 110 experts
    in use, the busiest with 488 rows."""
    logits = randn((tokens, experts), seed, "fp32")
    if skew:
        logits = logits - skew * torch.log1p(torch.arange(experts, dtype=torch.float32))
    probs = torch.softmax(logits, dim=-1)
    expert_of = torch.topk(probs, topk, dim=-1).indices            # [T, k]
    token_of = torch.arange(tokens).unsqueeze(1).expand(-1, topk)  # [T, k]
    key = (expert_of * tokens + token_of).reshape(-1)
    order = torch.argsort(key, stable=True)
    row_token = token_of.reshape(-1)[order]
    row_expert = expert_of.reshape(-1)[order]
    counts = torch.bincount(row_expert, minlength=experts)
    m_offsets = torch.zeros(experts + 1, dtype=torch.int32)
    m_offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
    return MoeRouting(expert_of, row_token, m_offsets)


def ragged_offsets(counts) -> torch.Tensor:
    """m_offsets int32[G+1] from per-group row counts (any counts, zeros allowed)."""
    c = torch.as_tensor(list(counts), dtype=torch.int64)
    off = torch.zeros(len(c) + 1, dtype=torch.int32)
    off[1:] = torch.cumsum(c, 0).to(torch.int32)
    return off
