"""Seeded synthetic inputs for the fused reduce + residual + RMSNorm (+fp8) epilogue.

This module holds shapes, value distributions and random draws only: none of the
method's arithmetic. Both the oracle side and the HIP side receive exactly the arrays
produced here.

Random numbers come from a counter-based generator, so that any element can be drawn on
its own and the values are the same on the CPU and on the GPU: element n of stream s is
the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) applied to seed + phi * (c + 1), with c = (s << 40) | n
and phi = 0x9E3779B97F4A7C15, all modulo 2^64.
  * uniform u = (x >> 11) * 2^-53, in [0, 1);
  * normal: Box-Muller on the pairs (2k, 2k+1) in fp64, r = sqrt(-2 ln(1 - u_2k)),
    z_2k = r cos(2 pi u_2k+1), z_2k+1 = r sin(2 pi u_2k+1).
Recipe (each workload is one of the five named below):
  * partials  [N][T][H]: stream 0 over the flattened array, normal(0, std) in fp64. With
    outliers, round(outlier_frac * H) hidden channels (stream 3: a partial Fisher-Yates
    shuffle of 0..H-1) are multiplied by ``outlier_scale`` in fp64 in every shard and
    token. Then rounded to fp32 and, for 16-bit partials, from fp32 to the partial type.
  * residual  [T][H]: stream 1, normal(0, residual_std), cast the same way.
  * gamma     [H]:    stream 2, 0.5 + u, cast the same way.
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


_PHI = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _signed(u: int) -> int:
    """A 64-bit pattern as the int64 value with the same bits."""
    return u - (1 << 64) if u >= 1 << 63 else u


def _srl(x: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns (torch's >> is arithmetic)."""
    return (x >> k) & ((1 << (64 - k)) - 1)


def raw64(seed: int, stream: int, start: int, count: int, device) -> torch.Tensor:
    """Elements start .. start+count-1 of a stream, as int64 bit patterns. int64 products
    wrap modulo 2^64 on both devices, which is the generator's arithmetic."""
    c = torch.arange(start, start + count, dtype=torch.int64, device=device) | (stream << 40)
    z = (c + 1) * _signed(_PHI) + _signed(seed & _MASK64)
    z = (z ^ _srl(z, 30)) * _signed(_MIX1)
    z = (z ^ _srl(z, 27)) * _signed(_MIX2)
    return z ^ _srl(z, 31)


def raw64_reference(seed: int, stream: int, n: int) -> int:
    """One element with Python integers, for checking raw64."""
    z = (seed + _PHI * (((stream << 40) | n) + 1)) & _MASK64
    z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
    z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
    return z ^ (z >> 31)


def uniform(seed: int, stream: int, start: int, count: int, device) -> torch.Tensor:
    """fp64 uniforms in [0, 1)."""
    return _srl(raw64(seed, stream, start, count, device), 11).to(torch.float64) * 2.0 ** -53


def normal(seed: int, stream: int, start: int, count: int, device) -> torch.Tensor:
    """fp64 standard normals; start and count are even (Box-Muller pairs)."""
    assert start % 2 == 0 and count % 2 == 0
    u = uniform(seed, stream, start, count, device).view(-1, 2)
    r = torch.sqrt(-2.0 * torch.log(1.0 - u[:, 0]))
    t = (2.0 * math.pi) * u[:, 1]
    return torch.stack((r * torch.cos(t), r * torch.sin(t)), dim=1).view(-1)


def outlier_channels(w: Workload) -> torch.Tensor:
    """Sorted indices of the hidden channels that carry outliers (CPU int64): the first
    round(outlier_frac * H) entries of a Fisher-Yates shuffle of 0..H-1 drawn from
    stream 3."""
    k = int(round(w.outlier_frac * w.hidden))
    if k == 0:
        return torch.empty(0, dtype=torch.int64)
    perm = list(range(w.hidden))
    draws = raw64(w.seed, 3, 0, k, "cpu").tolist()
    for i in range(k):
        j = i + (draws[i] & _MASK64) % (w.hidden - i)
        perm[i], perm[j] = perm[j], perm[i]
    return torch.sort(torch.tensor(perm[:k], dtype=torch.int64)).values


def _store(x64: torch.Tensor, dtype) -> torch.Tensor:
    x = x64.to(torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def generate_rows(w: Workload, row_begin: int, row_count: int, device="cpu"):
    """Rows row_begin .. row_begin+row_count-1 of the workload: (partials [N][count][H],
    residual [count][H], gamma [H]) on ``device``, the same values that ``generate`` puts in
    those rows (element (r, t, i) of the partials is element (r*T + t)*H + i of stream 0)."""
    device = torch.device(device)
    pdt, adt = TORCH_DTYPES[w.partial_dtype], TORCH_DTYPES[w.act_dtype]
    n, t, h = w.n_shards, w.tokens, w.hidden
    assert 0 <= row_begin and row_begin + row_count <= t
    partials = torch.empty((n, row_count, h), dtype=pdt, device=device)
    cols = outlier_channels(w).to(device)
    for r in range(n):  # one shard at a time bounds the fp64 temporaries
        x = normal(w.seed, 0, (r * t + row_begin) * h, row_count * h,
                   device).view(row_count, h).mul_(w.partial_std)
        if cols.numel():
            x[:, cols] *= w.outlier_scale
        partials[r].copy_(_store(x, pdt))
        del x
    res = _store(normal(w.seed, 1, row_begin * h, row_count * h,
                        device).view(row_count, h) * w.residual_std, adt)
    gamma = _store(uniform(w.seed, 2, 0, h, device) + 0.5, adt)
    return partials, res, gamma


def generate(w: Workload, device="cpu"):
    """Return (partials [N][T][H], residual [T][H], gamma [H]) as torch tensors on
    ``device`` in the workload's types; the same values on every device."""
    return generate_rows(w, 0, w.tokens, device)


def to_bits(x: torch.Tensor):
    """Host numpy view of a tensor: uint16 bit patterns for 16-bit types, float32 as is."""
    x = x.detach().to("cpu").contiguous()
    if x.dtype in (torch.bfloat16, torch.float16):
        return x.view(torch.int16).numpy().view("uint16")
    return x.numpy()
