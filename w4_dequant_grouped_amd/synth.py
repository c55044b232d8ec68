"""Seeded synthetic inputs for the W4 mixture-of-experts block.

This module only draws tensors: it holds none of the block's arithmetic (no
dequantisation, no routing, no matrix products).  Both the CPU oracle (under
``oracle/``) and the HIP path take their inputs from here, so the two sides see
bit-identical data.  Random draws use torch generators seeded explicitly, on
whatever device the caller names; a CPU draw and a GPU draw with the same seed
give different (but identically distributed) values.

Shapes follow the pages' model: 256 routed experts with eight selected per token
plus one shared expert ("Perplexity's Lily brings fast local AI to Apple silicon
Macs", section "A 35B Model Built for Local Memory"; "Perplexity built an
inference engine for one model, one chip", paragraph 2).  The pages give no
hidden size, intermediate size or group size; the workloads below fix them.

Weight format (the pages say only "groupwise affine 4-bit"):
  codes   uint8 [E][N][K/2]  two 4-bit codes per byte, K contiguous; byte j of a
                             row holds k = 2j in bits 0..3 and k = 2j+1 in bits 4..7
  scales  bf16  [E][N][K/G]  one scale per (row, group of G consecutive k)
  biases  bf16  [E][N][K/G]  one bias per (row, group)
Value distributions: codes uniform on 0..15 (uniform random bytes), scale drawn
U(0.005, 0.02) then rounded to bf16, bias = bf16(-8 * scale + N(0, 1e-3)) built
from the rounded scale; router weight fp32 N(0, 0.05); activations bf16(N(0, 1)).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

GROUP = 64


@dataclass(frozen=True)
class BlockShape:
    """Sizes of one MoE block call."""

    T: int          # tokens (rows of x)
    H: int          # hidden size
    I: int          # expert intermediate size (routed and shared)
    E: int          # routed experts
    top_k: int      # experts selected per token
    group: int = GROUP
    shared: bool = True
    router_bias: str = "none"   # "none" or "zipf"


@dataclass(frozen=True)
class Workload:
    name: str
    shape: BlockShape
    seed: int
    layers: int = 1
    note: str = ""


# Named workloads.  Seeds: the tiny block uses 0; the others use their index.
WORKLOADS = {
    "tiny": Workload("tiny", BlockShape(T=16, H=256, I=128, E=16, top_k=2), seed=0,
                     note="T=16, hidden 256, 16 experts top-2 + shared, intermediate 128"),
    "decode": Workload("decode", BlockShape(T=1, H=2048, I=512, E=256, top_k=8), seed=1,
                       note="T=1 (also T=2..5 verification rows), hidden 2048, 256 experts "
                            "top-8 + shared, intermediate 512"),
    "prefill512": Workload("prefill512", BlockShape(T=512, H=2048, I=512, E=256, top_k=8),
                           seed=2, note="T=512 prefill, uniform-ish routing"),
    "prefill2048_zipf": Workload("prefill2048_zipf",
                                 BlockShape(T=2048, H=2048, I=512, E=256, top_k=8,
                                            router_bias="zipf"),
                                 seed=3, note="T=2048 prefill, Zipf-skewed expert loads"),
    "stack40": Workload("stack40", BlockShape(T=16384, H=2048, I=512, E=256, top_k=8,
                                              router_bias="zipf"),
                        seed=4, layers=40, note="40 independent layers, T=16384 prefill + T=1 decode"),
}

ZIPF_S = 1.1      # exponent of the Zipf law behind the router bias
ZIPF_ALPHA = 1.5  # logit multiplier that makes some experts empty at T=2048


@dataclass
class W4Mat:
    """Packed 4-bit weights of E matrices of shape [N, K]."""

    codes: torch.Tensor    # uint8 [E, N, K // 2]
    scales: torch.Tensor   # bfloat16 [E, N, K // G]
    biases: torch.Tensor   # bfloat16 [E, N, K // G]

    def to(self, device) -> "W4Mat":
        return W4Mat(self.codes.to(device), self.scales.to(device), self.biases.to(device))

    def expert(self, e: int) -> "W4Mat":
        return W4Mat(self.codes[e:e + 1], self.scales[e:e + 1], self.biases[e:e + 1])


@dataclass
class Experts:
    """gate [E, I, H], up [E, I, H], down [E, H, I] in W4 form."""

    gate: W4Mat
    up: W4Mat
    down: W4Mat

    def to(self, device) -> "Experts":
        return Experts(self.gate.to(device), self.up.to(device), self.down.to(device))

    @property
    def num_experts(self) -> int:
        return self.gate.codes.shape[0]


@dataclass
class Layer:
    routed: Experts
    shared: Optional[Experts]         # one expert, or None
    router_w: torch.Tensor            # float32 [E, H]
    router_b: Optional[torch.Tensor]  # float32 [E] or None

    def to(self, device) -> "Layer":
        return Layer(self.routed.to(device),
                     None if self.shared is None else self.shared.to(device),
                     self.router_w.to(device),
                     None if self.router_b is None else self.router_b.to(device))


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    return g


def draw_w4(gen: torch.Generator, E: int, N: int, K: int, group: int = GROUP,
            device="cpu") -> W4Mat:
    assert K % group == 0 and K % 2 == 0
    codes = torch.randint(0, 256, (E, N, K // 2), dtype=torch.uint8, generator=gen, device=device)
    ng = K // group
    scale = torch.empty((E, N, ng), dtype=torch.float32, device=device).uniform_(
        0.005, 0.02, generator=gen).to(torch.bfloat16)
    noise = torch.randn((E, N, ng), dtype=torch.float32, generator=gen, device=device) * 1e-3
    bias = (-8.0 * scale.float() + noise).to(torch.bfloat16)
    return W4Mat(codes, scale, bias)


def draw_experts(gen: torch.Generator, E: int, H: int, I: int, group: int = GROUP,
                 device="cpu") -> Experts:
    gate = draw_w4(gen, E, I, H, group, device)
    up = draw_w4(gen, E, I, H, group, device)
    down = draw_w4(gen, E, H, I, group, device)
    return Experts(gate, up, down)


def zipf_router_bias(E: int, seed: int, alpha: float = ZIPF_ALPHA, s: float = ZIPF_S,
                     device="cpu") -> torch.Tensor:
    """Additive per-expert router bias -alpha * s * ln(rank), ranks a seeded permutation of 1..E."""
    g = generator(seed * 7919 + 17)
    rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
    return (-alpha * s * torch.log(rank)).to(torch.float32).to(device)


def _draw_router_w(gen: torch.Generator, shape: BlockShape, device) -> torch.Tensor:
    return torch.randn((shape.E, shape.H), dtype=torch.float32, generator=gen, device=device) * 0.05


def draw_router(shape: BlockShape, seed: int, device="cpu"):
    """The router weight and bias that ``draw_layer`` would draw, without the experts."""
    router_w = _draw_router_w(generator(seed, device), shape, device)
    router_b = zipf_router_bias(shape.E, seed, device=device) if shape.router_bias == "zipf" else None
    return router_w, router_b


def draw_layer(shape: BlockShape, seed: int, device="cpu") -> Layer:
    gen = generator(seed, device)
    router_w = _draw_router_w(gen, shape, device)
    routed = draw_experts(gen, shape.E, shape.H, shape.I, shape.group, device)
    shared = draw_experts(gen, 1, shape.H, shape.I, shape.group, device) if shape.shared else None
    router_b = zipf_router_bias(shape.E, seed, device=device) if shape.router_bias == "zipf" else None
    return Layer(routed, shared, router_w, router_b)


def _row_seed(seed: int, t: int, attempt: int) -> int:
    return (seed * 0x9E3779B1 + (t + 1) * 0x85EBCA77 + attempt * 0xC2B2AE3D) & ((1 << 62) - 1)


def draw_x(T: int, H: int, seed: int, device="cpu", redraws: Optional[dict] = None) -> torch.Tensor:
    """Activations bf16(N(0, 1)) of shape [T, H].

    ``redraws`` maps a row index to an attempt number >= 1; such a row is drawn
    again from its own sub-seed (seed, row, attempt) instead of the base stream.
    """
    x = torch.randn((T, H), dtype=torch.float32, generator=generator(seed + 0x5EED, device),
                    device=device)
    for t, attempt in (redraws or {}).items():
        if attempt:
            g = generator(_row_seed(seed, t, attempt), device)
            x[t] = torch.randn((H,), dtype=torch.float32, generator=g, device=device)
    return x.to(torch.bfloat16)


def block_bytes(shape: BlockShape) -> dict:
    """Sizes in bytes of the packed weights of one block (for bandwidth accounting)."""
    def mat(N, K):
        return N * K // 2 + 2 * 2 * N * (K // shape.group)
    per_expert = 2 * mat(shape.I, shape.H) + mat(shape.H, shape.I)
    return {
        "per_expert": per_expert,
        "router": shape.E * shape.H * 4 + (shape.E * 4 if shape.router_bias != "none" else 0),
        "layer": per_expert * (shape.E + (1 if shape.shared else 0)) + shape.E * shape.H * 4,
    }


def describe(shape: BlockShape) -> str:
    return (f"T={shape.T} H={shape.H} I={shape.I} E={shape.E} top{shape.top_k} "
            f"G={shape.group} shared={int(shape.shared)} bias={shape.router_bias}")


__all__ = [
    "GROUP", "BlockShape", "Workload", "WORKLOADS", "W4Mat", "Experts", "Layer", "generator",
    "draw_w4", "draw_experts", "draw_layer", "draw_router", "draw_x", "zipf_router_bias", "block_bytes",
    "describe", "ZIPF_S", "ZIPF_ALPHA",
]
