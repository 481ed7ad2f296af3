"""Seeded synthetic inputs for the INT4 KV-cache decode workloads.

This module only draws random numbers and describes workload shapes; it holds none of the
method's arithmetic.  It serves both the HIP path and the CPU oracle: both consume the same
tensors (the oracle gets host copies of bf16 bit patterns).

Workloads (decode shapes of Qwen3-8B / Qwen3-4B attention layers; the pages evaluate on those
models, whose weights and benchmark suites are not used here -- these draws stand in for them):
  tiny            1 sequence, 1 kv head, 2 q heads, D 64, 300 positions, S 4, R 32, b 32;
                  K, V ~ N(0,1) with 2 fixed K channels x20; q ~ N(0,1); seed 0
  qwen3_8b_layer  batch 64, lengths uniform in [1024, 8192], 32 q / 8 kv heads, D 128,
                  S 4, R 128, b 128; K ~ N(0,1) with 4 fixed channels per kv head x10, V ~ N(0,1)
  append          same shapes; 256 sequences x 512 single-position steps, and one bulk
                  prefill of 32768 positions into one sequence
  rollout         batch 256, lengths lognormal (median 4096, sigma 1.0) clipped to [256, 32768],
                  one step = 36 identical-shape layers, each with its own K/V draws
  long_context    batch 8, 131072 positions each, Qwen3-4B attention shapes (32 q / 8 kv, D 128)
All values are drawn in fp32 and rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_sinks: int
    num_recent: int
    hadamard_block: int
    batch: int
    outlier_channels: int
    outlier_scale: float
    seed: int = 0
    layers: int = 1
    lengths_kind: str = "fixed"
    length_args: tuple = ()
    page_size: int = 16

    def lengths(self) -> List[int]:
        rng = np.random.Generator(np.random.PCG64(self.seed + 7919))
        if self.lengths_kind == "fixed":
            return [int(self.length_args[0])] * self.batch
        if self.lengths_kind == "uniform":
            lo, hi = self.length_args
            return [int(x) for x in rng.integers(lo, hi + 1, size=self.batch)]
        if self.lengths_kind == "lognormal":
            median, sigma, lo, hi = self.length_args
            x = np.exp(math.log(median) + sigma * rng.standard_normal(self.batch))
            return [int(min(max(round(v), lo), hi)) for v in x]
        raise ValueError(self.lengths_kind)


WORKLOADS = {
    "tiny": Workload("tiny", 2, 1, 64, 4, 32, 32, 1, 2, 20.0, lengths_kind="fixed", length_args=(300,)),
    "qwen3_8b_layer": Workload("qwen3_8b_layer", 32, 8, 128, 4, 128, 128, 64, 4, 10.0, lengths_kind="uniform",
                               length_args=(1024, 8192)),
    "append": Workload("append", 32, 8, 128, 4, 128, 128, 256, 4, 10.0, lengths_kind="fixed", length_args=(512,)),
    "rollout": Workload("rollout", 32, 8, 128, 4, 128, 128, 256, 4, 10.0, layers=36, lengths_kind="lognormal",
                        length_args=(4096, 1.0, 256, 32768)),
    "long_context": Workload("long_context", 32, 8, 128, 4, 128, 128, 8, 4, 10.0, lengths_kind="fixed",
                             length_args=(131072,)),
    # one GPU's share of the rollout regime under 8-way tensor parallelism by kv head: the same
    # sequences and lengths, 1 kv head and its 4 query heads
    "rollout_tp8": Workload("rollout_tp8", 4, 1, 128, 4, 128, 128, 256, 4, 10.0, layers=36, lengths_kind="lognormal",
                            length_args=(4096, 1.0, 256, 32768)),
}


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from integers (splitmix64 steps)."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x = (x ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


def outlier_channels(num_kv_heads: int, head_dim: int, count: int, seed: int, layer: int = 0) -> np.ndarray:
    """Fixed outlier channels per kv head: [num_kv_heads][count] distinct indices."""
    rng = np.random.Generator(np.random.PCG64(_mix(seed, layer, 17)))
    return np.stack([rng.choice(head_dim, size=count, replace=False) for _ in range(num_kv_heads)]).astype(np.int64)


def _generator(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def seq_kv(num_kv_heads: int, head_dim: int, length: int, channels: np.ndarray, scale: float, seed: int, layer: int,
           seq_index: int, device="cpu"):
    """K, V bf16 [length, Hkv, D] for one sequence of one layer.  K has `channels` scaled by `scale`."""
    device = torch.device(device)
    g = _generator(device, _mix(seed, layer, seq_index, 1))
    k = torch.randn((length, num_kv_heads, head_dim), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((length, num_kv_heads, head_dim), generator=g, device=device, dtype=torch.float32)
    if channels is not None and channels.size:
        mult = torch.ones((num_kv_heads, head_dim), dtype=torch.float32)
        for h in range(num_kv_heads):
            mult[h, torch.as_tensor(channels[h])] = scale
        k = k * mult.to(device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def queries(n: int, num_q_heads: int, head_dim: int, seed: int, layer: int = 0, step: int = 0, device="cpu"):
    """q bf16 [n, Hq, D] ~ N(0, 1)."""
    device = torch.device(device)
    g = _generator(device, _mix(seed, layer, step, 2))
    return torch.randn((n, num_q_heads, head_dim), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 bit patterns of a bf16 tensor."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rope_tables(positions: int, head_dim: int, base: float = 1.0e6):
    """Standard rotary-embedding tables (the caller's data for the fused RoPE append): float32
    cos / sin [positions, head_dim / 2] of angle t * base^(-2i / head_dim), computed in float64.
    base 1e6 is Qwen3's."""
    inv = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def tiny_inputs(device="cpu"):
    """The tiny workload: (K, V [300, 1, 64], q [1, 2, 64]) with seed 0."""
    w = WORKLOADS["tiny"]
    ch = outlier_channels(w.num_kv_heads, w.head_dim, w.outlier_channels, w.seed)
    k, v = seq_kv(w.num_kv_heads, w.head_dim, 300, ch, w.outlier_scale, w.seed, 0, 0, device)
    q = queries(1, w.num_q_heads, w.head_dim, w.seed, device=device)
    return k, v, q
