"""Seeded synthetic inputs for the fused reduce + residual + RMSNorm (+fp8) epilogue.

This module holds shapes, value distributions and random draws only: none of the
method's arithmetic. Both the oracle side and the HIP side receive exactly the arrays
produced here.

Recipe (each workload is one of the five named below):
  * partials  [N][T][H]: normal(0, std) drawn in fp32, then cast (round-to-nearest-even,
    torch's own cast) to the partial type. With outliers, a seeded choice of
    round(outlier_frac * H) hidden channels is multiplied by ``outlier_scale`` in fp32 in
    every shard and token before the cast.
  * residual  [T][H]: normal(0, residual_std) in fp32, cast to the activation type.
  * gamma     [H]:    uniform(0.5, 1.5) in fp32, cast to the activation type.
Each of the four draws uses its own torch.Generator seeded with seed*16 + stream
(stream 0 partials, 1 residual, 2 gamma, 3 outlier channels). The outlier channel choice
always uses a CPU generator. For a given (workload, device type) the values are
reproducible; CPU and GPU generators produce different streams, so a test that checks a
GPU run copies the generated inputs to the host for the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    n_shards: int
    tokens: int
    hidden: int
    partial_dtype: str          # "bf16" | "f16" | "f32"
    act_dtype: str              # "bf16" | "f16"
    partial_std: float
    residual_std: float
    eps: float
    quant: str | None           # None | "per_tensor" | "per_token"
    seed: int
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    @property
    def sp(self) -> int:
        return 4 if self.partial_dtype == "f32" else 2

    @property
    def sa(self) -> int:
        return 2

    def algorithmic_bytes(self) -> int:
        """Each input read once, each output written once (residual_out and norm_out are
        always written; fp8 codes and the scale when quantising)."""
        n, t, h = self.n_shards, self.tokens, self.hidden
        b = n * t * h * self.sp + t * h * self.sa + h * self.sa + 2 * t * h * self.sa
        if self.quant == "per_tensor":
            b += t * h + 4
        elif self.quant == "per_token":
            b += t * h + 4 * t
        return b

    def with_tokens(self, tokens: int) -> "Workload":
        return replace(self, tokens=tokens)


# The five workloads. Distributions: "N(0, s)" is read as standard deviation s.
WORKLOADS = {
    # N=2, 16 tokens, hidden 1024, bf16; partials N(0,1)/sqrt(N).
    "c0": Workload("c0_n2_t16_h1024_bf16", 2, 16, 1024, "bf16", "bf16",
                   1.0 / math.sqrt(2.0), 1.0, 1e-6, None, 0),
    # N=8, 128 tokens, hidden 4096 (Llama-8B-like), bf16; partials N(0,0.5).
    "c1": Workload("c1_n8_t128_h4096_bf16", 8, 128, 4096, "bf16", "bf16",
                   0.5, 1.0, 1e-5, None, 1),
    # N=8, 64 decode tokens, hidden 8192, bf16; same distributions; per-tensor fp8 copy.
    "c2": Workload("c2_n8_t64_h8192_bf16_fp8tensor", 8, 64, 8192, "bf16", "bf16",
                   0.5, 1.0, 1e-5, "per_tensor", 2),
    # N=4 fp32 partials, 2048 prefill tokens, hidden 7168, bf16 activations; 1% of the
    # hidden channels carry x100 outliers.
    "c3": Workload("c3_n4_t2048_h7168_f32partials", 4, 2048, 7168, "f32", "bf16",
                   1.0, 1.0, 1e-6, None, 3, outlier_frac=0.01, outlier_scale=100.0),
    # N=8, 8192 tokens, hidden 16384, bf16 (2 GiB of partials); per-token fp8 copy.
    "c4": Workload("c4_n8_t8192_h16384_bf16_fp8token", 8, 8192, 16384, "bf16", "bf16",
                   1.0, 1.0, 1e-6, "per_token", 4),
}


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + stream)
    return g


def outlier_channels(w: Workload) -> torch.Tensor:
    """Sorted indices of the hidden channels that carry outliers (CPU int64)."""
    k = int(round(w.outlier_frac * w.hidden))
    if k == 0:
        return torch.empty(0, dtype=torch.int64)
    perm = torch.randperm(w.hidden, generator=_gen(w.seed, 3, "cpu"))
    return torch.sort(perm[:k]).values


def generate(w: Workload, device="cpu"):
    """Return (partials [N][T][H], residual [T][H], gamma [H]) as torch tensors on
    ``device`` in the workload's types."""
    device = torch.device(device)
    pdt, adt = TORCH_DTYPES[w.partial_dtype], TORCH_DTYPES[w.act_dtype]
    n, t, h = w.n_shards, w.tokens, w.hidden
    gp = _gen(w.seed, 0, device)
    partials = torch.empty((n, t, h), dtype=pdt, device=device)
    cols = outlier_channels(w).to(device)
    for r in range(n):  # one shard at a time bounds the fp32 temporary
        x = torch.randn((t, h), generator=gp, device=device, dtype=torch.float32)
        x.mul_(w.partial_std)
        if cols.numel():
            x[:, cols] *= w.outlier_scale
        partials[r].copy_(x)
        del x
    res = torch.randn((t, h), generator=_gen(w.seed, 1, device), device=device,
                      dtype=torch.float32).mul_(w.residual_std).to(adt)
    gamma = (torch.rand((h,), generator=_gen(w.seed, 2, device), device=device,
                        dtype=torch.float32) + 0.5).to(adt)
    return partials, res, gamma


def to_bits(x: torch.Tensor):
    """Host numpy view of a tensor: uint16 bit patterns for 16-bit types, float32 as is."""
    x = x.detach().to("cpu").contiguous()
    if x.dtype in (torch.bfloat16, torch.float16):
        return x.view(torch.int16).numpy().view("uint16")
    return x.numpy()
