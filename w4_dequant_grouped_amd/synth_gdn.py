"""Seeded synthetic inputs for the Gated DeltaNet scan of the linear-attention layers.

This module only draws tensors: it holds none of the scan's arithmetic.  The CPU
oracle under ``oracle/`` and the HIP path take their inputs from here.

Thirty of the model's 40 layers run Gated DeltaNet, which keeps a fixed-size
recurrent state per head instead of a growing cache ("Perplexity built an
inference engine for one model, one chip", paragraph 2), and the engine's prefill
gained from keeping that state in registers during the scan ("Perplexity's Lily
brings fast local AI to Apple silicon Macs", section "Where the Engine Gains
Speed").  The pages give no head counts or sizes; the shapes below take 32 value
heads over 16 query/key heads of dimension 128.

Layout (row-major):
  q, k    bf16  [T][Hk][128]   unit-norm rows (the layer normalises them before the scan)
  v       bf16  [T][Hv][128]
  g       fp32  [T][Hv]        log of the decay, g <= 0 (alpha = exp(g))
  beta    fp32  [T][Hv]        write strength in (0, 1)
  state   fp32  [Hv][128][128] state[h][i][j]: value row i, key column j
Value head h reads query/key head h // (Hv / Hk).
Values: q, k = bf16 of normalised N(0, I) draws (renormalised after rounding is not
attempted: the bf16 rows are within 2^-8 of unit norm); v = bf16(N(0, 1));
g = log(U(0.90, 1.0)); beta = U(0.05, 0.95); the initial state N(0, 0.1^2).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from .synth import generator


@dataclass(frozen=True)
class GdnShape:
    T: int
    n_v_heads: int = 32
    n_k_heads: int = 16
    dim: int = 128


@dataclass
class GdnInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    state: torch.Tensor

    def to(self, device) -> "GdnInputs":
        return GdnInputs(*(t.to(device) for t in (self.q, self.k, self.v, self.g, self.beta, self.state)))


GDN_WORKLOADS = {
    "tiny": (GdnShape(T=70, n_v_heads=4, n_k_heads=2), 20),
    "decode": (GdnShape(T=1), 21),
    "prefill512": (GdnShape(T=512), 22),
    "prefill2048": (GdnShape(T=2048), 23),
}


def draw_gdn(shape: GdnShape, seed: int, device="cpu") -> GdnInputs:
    gen = generator(seed * 104729 + 0x6D1, device)
    T, Hv, Hk, d = shape.T, shape.n_v_heads, shape.n_k_heads, shape.dim
    q = torch.randn((T, Hk, d), generator=gen, device=device)
    k = torch.randn((T, Hk, d), generator=gen, device=device)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((T, Hv, d), generator=gen, device=device)
    alpha = 0.90 + 0.10 * torch.rand((T, Hv), generator=gen, device=device)
    g = torch.log(alpha)
    beta = 0.05 + 0.90 * torch.rand((T, Hv), generator=gen, device=device)
    state = 0.1 * torch.randn((Hv, d, d), generator=gen, device=device)
    return GdnInputs(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16),
                     g.float(), beta.float(), state.float())


def gdn_bytes(shape: GdnShape) -> int:
    """Bytes one scan reads or writes once: inputs, outputs, state in and out."""
    T, Hv, Hk, d = shape.T, shape.n_v_heads, shape.n_k_heads, shape.dim
    return (2 * T * Hk * d * 2 + T * Hv * d * 2 + 2 * T * Hv * 4 + T * Hv * d * 2
            + 2 * Hv * d * d * 4)


def gdn_flops(shape: GdnShape) -> int:
    """fp32 operations per scan: per token, value row and key column, the two dots
    (S k, S q) and the rank-one update (a multiply-add each): 6 flops."""
    return 6 * shape.T * shape.n_v_heads * shape.dim * shape.dim
