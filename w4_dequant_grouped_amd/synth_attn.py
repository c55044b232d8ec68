"""Seeded synthetic inputs for one decode-attention step over a paged KV cache.

This module only draws tensors: it holds none of the attention arithmetic (no
products, no softmax).  The CPU oracle under ``oracle/`` and the HIP path take
their inputs from here, so both see bit-identical data.

The step is the decode side of the model's full-attention layers: one new query
token attends to every cached token.  The pages give the head layout (16 query
heads sharing two key/value heads: "Perplexity's Lily brings fast local AI to
Apple silicon Macs", section "A 35B Model Built for Local Memory") and the
context lengths of interest (32K to 128K: the same page, section "Where the
Engine Gains Speed"), and describe the cache as read in fixed-size blocks.  They
give no head dimension or block size; the shapes below fix them (128 and 64).

Layout (the "fixed-block" reading):
  q         bf16  [Hq][d]                       the new token's query heads
  k_pool    bf16  [P][Hkv][B][d]                P physical blocks of B tokens
  v_pool    bf16  [P][Hkv][B][d]
  table     int32 [ceil(n_ctx / B)]             logical block i lives in physical
                                                block table[i]; token n is slot
                                                n % B of logical block n // B
Query head h reads key/value head h // (Hq / Hkv).
Values: q, K, V bf16(N(0, 1)); the table is a seeded draw of distinct physical
blocks (the pool holds a few spare blocks that no table entry names).  Slots past
n_ctx in the last block and the spare blocks hold ordinary draws, or NaN when
``poison_tail`` is set, so that a reader of anything outside the context shows.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from .synth import generator


@dataclass(frozen=True)
class AttnShape:
    n_ctx: int              # cached tokens the query attends to (>= 1)
    n_q_heads: int = 16
    n_kv_heads: int = 2
    head_dim: int = 128
    block: int = 64         # tokens per KV block
    spare_blocks: int = 3   # physical blocks no table entry names
    poison_tail: bool = False

    @property
    def n_blocks(self) -> int:
        return math.ceil(self.n_ctx / self.block)

    @property
    def n_pool_blocks(self) -> int:
        return self.n_blocks + self.spare_blocks


@dataclass
class AttnInputs:
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    table: torch.Tensor

    def to(self, device) -> "AttnInputs":
        return AttnInputs(*(t.to(device) for t in (self.q, self.k_pool, self.v_pool, self.table)))


ATTN_WORKLOADS = {
    "tiny": (AttnShape(n_ctx=300, n_q_heads=16, n_kv_heads=2), 10),
    "ctx32k": (AttnShape(n_ctx=32768), 11),
    "ctx64k": (AttnShape(n_ctx=65536), 12),
    "ctx128k": (AttnShape(n_ctx=131072), 13),
}


def draw_attn(shape: AttnShape, seed: int, device="cpu") -> AttnInputs:
    """q, k_pool, v_pool and the block table of one decode-attention step."""
    g = generator(seed * 7919 + 0xA77, device)
    P, Hkv, B, d = shape.n_pool_blocks, shape.n_kv_heads, shape.block, shape.head_dim
    q = torch.randn((shape.n_q_heads, d), generator=g, device=device)
    k = torch.randn((P, Hkv, B, d), generator=g, device=device)
    v = torch.randn((P, Hkv, B, d), generator=g, device=device)
    perm = torch.randperm(P, generator=g, device=device)
    table = perm[: shape.n_blocks].to(torch.int32)
    if shape.poison_tail:
        used = torch.zeros(P, dtype=torch.bool, device=device)
        used[table.long()] = True
        k[~used] = float("nan")
        v[~used] = float("nan")
        tail = shape.n_ctx - (shape.n_blocks - 1) * B      # valid slots of the last block
        if tail < B:
            last = int(table[-1])
            k[last, :, tail:] = float("nan")
            v[last, :, tail:] = float("nan")
    return AttnInputs(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), table)


def attn_bytes(shape: AttnShape) -> int:
    """Bytes one step must read or write once: the context's K and V rows, q, out."""
    kv = 2 * shape.n_ctx * shape.n_kv_heads * shape.head_dim * 2
    return kv + 2 * shape.n_q_heads * shape.head_dim * 2 + shape.n_blocks * 4
