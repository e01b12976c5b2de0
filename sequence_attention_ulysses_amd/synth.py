"""Seeded synthetic inputs shared by the HIP path, its tests and the benchmark.

This module draws random numbers and rounds them to the storage dtype; it
holds none of the exchange's or the norm/rotary arithmetic, so both the HIP
library and the CPU oracle can be fed from it.

Workload shapes are video-DiT attention blocks of the kind the pages run
(LingBot-World, Wan, MiniMax H3): values are N(0, 1) activations and
N(1, 0.1) RMSNorm weights, rounded once to bf16 or fp16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


def generator(seed: int, device: str | torch.device = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, dtype: str, seed: int, device="cpu", mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    """N(mean, std) drawn in fp32 from a seeded generator, rounded once to ``dtype``."""
    g = generator(seed, device)
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(DTYPES[dtype])


def norm_weight(D: int, dtype: str, seed: int, device="cpu") -> torch.Tensor:
    """A per-head RMSNorm weight [D] ~ N(1, 0.1) in the activation dtype."""
    return normal((D,), dtype, seed, device, mean=1.0, std=0.1)


def random_bytes(shape, seed: int, dtype: torch.dtype = torch.uint8, device="cpu") -> torch.Tensor:
    """Uniform random bytes viewed as a 1-byte dtype (fp8 / int8 payloads as opaque bits)."""
    g = generator(seed, "cpu")
    t = torch.randint(0, 256, tuple(shape), generator=g, dtype=torch.uint8)
    return t.view(dtype).to(device)


def bits(t: torch.Tensor):
    """Storage of a CPU tensor as numpy unsigned words: uint16 for 16-bit types (bf16
    has no numpy dtype), uint8 for 1-byte types."""
    if t.element_size() == 1:
        return t.contiguous().view(torch.uint8).numpy()
    return t.contiguous().view(torch.int16).numpy().view("uint16")


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity shape.  Per-rank tensors are stored rank-major."""

    name: str
    P: int
    B: int
    S_l: int          # per-rank sequence after padding
    Hq: int
    Hkv: int
    D: int
    dtype: str
    fused_qkv: bool = False      # V (and Q, K) taken from one [B, S_l, 3, H, D] tensor
    norm_rope: bool = False      # Q/K RMSNorm + RoPE fused into the scatter
    S_real: int | None = None    # global real tokens (padded sequences)
    rope: str = "1d"             # "1d" or "3d"
    grid: tuple = field(default=())   # (T, Hh, Ww) latent grid for 3-D RoPE
    theta: float = 1e4
    eps: float = 1e-6

    @property
    def S(self) -> int:
        return self.P * self.S_l

    @property
    def tokens(self) -> int:
        return self.S if self.S_real is None else self.S_real


# The five workloads: a tiny round trip, a video-DiT block with fused QKV,
# a Wan-style long sequence padded to a multiple of P*128, a GQA block and
# (separately, see SPATIAL) a height-sharded latent.
TINY = Workload("tiny_p2_f16", P=2, B=1, S_l=128, Hq=8, Hkv=8, D=64, dtype="f16")
VIDEO_DIT = Workload("video_dit_p4_s16384_h24_bf16", P=4, B=1, S_l=4096, Hq=24, Hkv=24, D=128,
                     dtype="bf16", fused_qkv=True, norm_rope=True)
WAN_LONG = Workload("wan_long_p4_s75600_h40_bf16", P=4, B=1, S_l=18944, Hq=40, Hkv=40, D=128,
                    dtype="bf16", norm_rope=True, S_real=75600, rope="3d", grid=(21, 60, 60))
GQA = Workload("gqa_p8_b2_s65536_hq32_hkv8_bf16", P=8, B=2, S_l=8192, Hq=32, Hkv=8, D=128,
               dtype="bf16")


@dataclass(frozen=True)
class SpatialWorkload:
    name: str
    P: int
    shape: tuple       # [B, C, T, Hh, W]
    dtype: str
    halo: int = 1


SPATIAL = SpatialWorkload("spatial_p4_latent_1x16x21x90x160_bf16", P=4, shape=(1, 16, 21, 90, 160),
                          dtype="bf16")

WORKLOADS = {w.name: w for w in (TINY, VIDEO_DIT, WAN_LONG, GQA)}
