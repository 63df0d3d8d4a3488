"""Seeded synthetic inputs for the KIVI hot path (keys, values, queries).

This module only draws random tensors; it holds none of the quantization or
attention arithmetic.  Tests feed the same tensors to the HIP library and to
the CPU oracle, and bench.py uses it for its workloads.

Distributions follow the outlier structure the pages describe: keys carry a
few channels of persistently large magnitude, values carry occasional tokens
with a burst over all channels (page "KIVI: Asymmetric 2-Bit KV Cache
Quantization Guide", section "Why Standard Uniform Quantization Fails on KV
Caches"; page "KV-Cache Quantization: I Ran the Experiments", "Component 2").

Draw order for one layer (all in float32, then rounded to nearest-even into
the storage dtype):
  1. outlier key channels per kv head (fixed across batch and tokens)
  2. per-(head, channel) key offset ~ N(0, 2)   (variance 2)
  3. K = z * (15 on outlier channels, else 1) + offset, z ~ N(0, 1)
  4. V = z * (8 on outlier tokens, else 1), outlier token ~ Bernoulli(0.01)
     per (batch, head, token)
  5. q ~ N(0, 1)
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    tokens: int              # prefix length T appended before the decode step
    k_bits: int
    v_bits: int
    dtype: torch.dtype       # storage dtype of K, V, q and the residual window
    outliers: Tuple[int, int]  # outlier key channels per head: U{lo..hi}
    layers: int = 1
    group_size: int = 32
    residual_length: int = 128
    description: str = ""

    @property
    def gq(self) -> int:
        return self.q_heads // self.kv_heads


# The five workload shapes (attention-layer shapes of Llama-2-7B, Llama-3-8B
# and Mistral-7B; these models are named on the pages, their weights are not
# used).  All use G = 32, R = 128 and softmax scale 1/sqrt(128).
WORKLOADS = {
    "c0": Workload("c0", 1, 1, 1, 128, 1024, 2, 2, torch.float16, (4, 4),
                   description="1 sequence, 1 kv head, T=1024 (896 packed + 128 "
                               "window), 2-bit, seed 0"),
    "c1": Workload("c1", 8, 32, 32, 128, 4096, 2, 2, torch.float16, (4, 4),
                   description="Llama-2-7B-shaped MHA layer, batch 8, T=4096, "
                               "2-bit: prefix pack plus one decode step"),
    "c2": Workload("c2", 32, 8, 32, 128, 32768, 2, 2, torch.float16, (2, 6),
                   description="Llama-3-8B-shaped GQA layer (32q/8kv), batch 32, "
                               "T=32768, 2-bit: window flush plus decode"),
    "c3": Workload("c3", 64, 8, 32, 128, 8192, 4, 4, torch.bfloat16, (4, 4),
                   description="Mistral-7B-shaped GQA layer, batch 64, T=8192, "
                               "4-bit, bf16: prefix pack plus one decode step"),
    "c4": Workload("c4", 4, 8, 32, 128, 131072, 2, 2, torch.float16, (4, 4),
                   layers=32,
                   description="Llama-3-8B-shaped GQA, batch 4, T=131072, 2-bit, "
                               "32 layers of one decode step"),
}


def small(name: str, batch: int, kv_heads: int, q_heads: int, tokens: int,
          k_bits: int = 2, v_bits: int = 2, dtype=torch.float16,
          head_dim: int = 128, residual_length: int = 128,
          outliers=(4, 4)) -> Workload:
    """A reduced workload with the same distributions (for parity tests)."""
    return Workload(name, batch, kv_heads, q_heads, head_dim, tokens, k_bits,
                    v_bits, dtype, outliers, residual_length=residual_length)


@dataclass
class LayerInputs:
    k: torch.Tensor          # [B][H][T + n_new][D] storage dtype
    v: torch.Tensor
    q: torch.Tensor          # [B][Hq][D] storage dtype
    outlier_channels: list = field(default_factory=list)


def make_layer(w: Workload, seed: int, device="cpu", n_new: int = 1,
               tokens: Optional[int] = None) -> LayerInputs:
    """Draws K/V for T (+ n_new decode tokens) positions and one query per
    query head.  Deterministic for a given (seed, device, torch version)."""
    T = (w.tokens if tokens is None else tokens) + n_new
    B, H, Hq, D = w.batch, w.kv_heads, w.q_heads, w.head_dim
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    lo, hi = w.outliers
    # 1. outlier channels per kv head
    key_gain = torch.ones(H, D, dtype=torch.float32, device=device)
    chans = []
    for h in range(H):
        n = int(torch.randint(lo, hi + 1, (1,), generator=g, device=device).item())
        perm = torch.randperm(D, generator=g, device=device)[:n]
        key_gain[h, perm] = 15.0
        chans.append(sorted(perm.tolist()))
    # 2. per-channel offsets ~ N(0, 2)
    offset = torch.randn(H, D, generator=g, device=device) * (2.0 ** 0.5)
    # 3. keys
    k = torch.randn(B, H, T, D, generator=g, device=device)
    k.mul_(key_gain[None, :, None, :]).add_(offset[None, :, None, :])
    k = k.to(w.dtype)
    # 4. values with 1% outlier tokens
    v = torch.randn(B, H, T, D, generator=g, device=device)
    mask = torch.rand(B, H, T, 1, generator=g, device=device) < 0.01
    v = torch.where(mask, v * 8.0, v).to(w.dtype)
    # 5. queries
    q = torch.randn(B, Hq, D, generator=g, device=device).to(w.dtype)
    return LayerInputs(k=k, v=v, q=q, outlier_channels=chans)


def bits16(t: torch.Tensor):
    """Raw 16-bit patterns of an fp16/bf16 tensor as a numpy uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
