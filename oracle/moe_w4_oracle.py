"""CPU oracle for the W4 mixture-of-experts block.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP path and never
calls it; its only shared dependency is the seeded input generator.

It is the plain definition of what the block computes, written out in float64
with NumPy, one step after another, with no blocking, fusion or reordering:

  1. dequantise every 4-bit weight to w = code * scale + bias  (groupwise affine
     4-bit quantisation: "Perplexity's Lily brings fast local AI to Apple silicon
     Macs", section "A 35B Model Built for Local Memory")
  2. router logits l = x W_r^T (+ b_r), softmax over all experts, keep the top-k
     (k = 8 of 256 at full size) and renormalise their probabilities ("Perplexity
     built an inference engine for one model, one chip", paragraph 2: a router
     picks eight subnetworks out of 256)
  3. group the (token, slot) pairs by expert: counts, offsets, token permutation
  4. per expert, a SwiGLU MLP silu(X Wg^T) * (X Wu^T) then Wd^T over its rows
     ("the grouped GEMM" of the same page, paragraph 3, and of "Perplexity's Lily
     brings fast local AI to Apple silicon Macs", section "Where the Engine Gains
     Speed"), weighted by the routing weight and added into the token's output
  5. the shared expert's SwiGLU MLP on every token, weight 1 ("one shared expert
     sees everything", "Perplexity built an inference engine for one model, one
     chip", paragraph 2)

Fusing the dequantisation into the GEMM and keeping routing on the GPU (the same
page, paragraph 3) change where the work happens, not its result, so the oracle
is the unfused definition.

Readings taken where the pages are silent:
nibble order (low nibble = even k), group size 64 along K, affine form
code*scale+bias with unsigned codes 0..15, softmax over all experts then top-k
then renormalise, ties broken towards the lower expert index, each token's ids
reported in ascending expert order, the permutation ordered by (expert, token),
the shared expert un-gated with weight 1, SwiGLU activation, output overwritten.

Parity is pinned by tests/test_oracle.py against hand-worked groups, exact
integer-valued logits, brute-force top-k, brute-force grouping, the textbook
dense SwiGLU MLP, closed-form special cases and invariants.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

try:  # tensors from the input generator are torch tensors; plain arrays work too
    import torch
except ImportError:  # pragma: no cover
    torch = None


# ----------------------------------------------------------------------------
# input decoding
# ----------------------------------------------------------------------------

def _as_numpy(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        a = a.detach().cpu()
        if a.dtype == torch.bfloat16:
            return a.view(torch.int16).numpy().view(np.uint16)
        return a.numpy()
    return np.asarray(a)


def bf16_to_f64(a) -> np.ndarray:
    """bfloat16 (given as a torch bf16 tensor or as uint16 bit patterns) to float64.

    A bf16 value is the upper half of a float32, so the conversion is exact.
    """
    bits = _as_numpy(a)
    assert bits.dtype == np.uint16, bits.dtype
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_f64(a) -> np.ndarray:
    arr = _as_numpy(a)
    assert arr.dtype == np.float32, arr.dtype
    return arr.astype(np.float64)


def unpack_codes(packed) -> np.ndarray:
    """uint8 [..., N, K/2] -> uint8 [..., N, K]: byte j holds k=2j (low) and k=2j+1 (high)."""
    p = _as_numpy(packed)
    assert p.dtype == np.uint8
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant(codes, scales, biases, group: int) -> np.ndarray:
    """W[..., n, k] = code[..., n, k] * scale[..., n, k // group] + bias[..., n, k // group].

    Groupwise affine 4-bit weights ("Perplexity's Lily brings fast local AI to
    Apple silicon Macs", section "A 35B Model Built for Local Memory").
    """
    c = unpack_codes(codes).astype(np.float64)
    s = bf16_to_f64(scales)
    b = bf16_to_f64(biases)
    K = c.shape[-1]
    assert s.shape[-1] * group == K and b.shape == s.shape
    g = np.arange(K) // group
    return c * s[..., g] + b[..., g]


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

@dataclass
class Routing:
    ids: np.ndarray        # int32 [T, k], ascending expert id per token
    weights: np.ndarray    # float64 [T, k], weight of ids[t, j]
    counts: np.ndarray     # int32 [E]
    offsets: np.ndarray    # int32 [E + 1], exclusive prefix sum of counts
    perm: np.ndarray       # int32 [T * k], (t * k + slot) ordered by (expert, t)
    logits: np.ndarray     # float64 [T, E]


def router_logits(x, router_w, router_b=None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * W_r[e, h] + b_r[e], in float64."""
    xf = bf16_to_f64(x)
    wr = f32_to_f64(router_w)
    l = xf @ wr.T
    if router_b is not None:
        l = l + f32_to_f64(router_b)[None, :]
    return l


def select_experts(logits: np.ndarray, top_k: int):
    """Softmax over all experts, top-k by logit (ties to the lower index), renormalise.

    Returns (ids ascending per token, their renormalised weights).
    """
    T, E = logits.shape
    assert 1 <= top_k <= E
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    for t in range(T):
        l = logits[t]
        p = np.exp(l - l.max())
        p = p / p.sum()                                  # softmax over all E experts
        order = sorted(range(E), key=lambda e: (-l[e], e))  # by logit, ties -> lower index
        chosen = sorted(order[:top_k])                   # report ascending expert id
        sel = p[chosen]
        ids[t] = chosen
        w[t] = sel / sel.sum()                           # renormalise over the chosen
    return ids, w


def group_by_expert(ids: np.ndarray, num_experts: int):
    """counts[e], offsets (exclusive scan, length E+1) and perm ordered by (expert, token)."""
    T, k = ids.shape
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in ids.ravel():
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm = np.empty(T * k, dtype=np.int64)
    # a stable sort of the flat (t * k + slot) indices by expert id; a token holds
    # an expert at most once, so within one expert this is token order
    flat = ids.ravel()
    for idx in np.argsort(flat, kind="stable"):
        e = flat[idx]
        perm[fill[e]] = idx
        fill[e] += 1
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32)


def route(x, router_w, router_b, top_k: int) -> Routing:
    l = router_logits(x, router_w, router_b)
    ids, w = select_experts(l, top_k)
    counts, offsets, perm = group_by_expert(ids, l.shape[1])
    return Routing(ids, w, counts, offsets, perm, l)


def kth_gap(logits: np.ndarray, top_k: int) -> np.ndarray:
    """Per token, the k-th largest logit minus the (k+1)-th (inf when k = E)."""
    T, E = logits.shape
    if top_k >= E:
        return np.full(T, np.inf)
    srt = -np.sort(-logits, axis=1)
    return srt[:, top_k - 1] - srt[:, top_k]


# ----------------------------------------------------------------------------
# expert MLPs
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_mlp(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """(silu(X Wg^T) * (X Wu^T)) Wd^T for X [M, H], Wg/Wu [I, H], Wd [H, I]."""
    return (silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T


class _ExpertCache:
    """Dequantises an expert's three matrices on first use."""

    def __init__(self, experts, group: int):
        self.experts = experts
        self.group = group
        self.cache = {}

    def __call__(self, e: int):
        if e not in self.cache:
            ex = self.experts
            self.cache[e] = tuple(
                dequant(m.codes[e], m.scales[e], m.biases[e], self.group)
                for m in (ex.gate, ex.up, ex.down))
        return self.cache[e]


def forward_grouped(x, layer, routing: Routing, group: int) -> np.ndarray:
    """Grouped form: for each expert, gather its rows, run its MLP, scatter-add weighted rows."""
    xf = bf16_to_f64(x)
    T, H = xf.shape
    k = routing.ids.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    E = routing.counts.shape[0]
    for e in range(E):
        lo, hi = int(routing.offsets[e]), int(routing.offsets[e + 1])
        if hi == lo:
            continue
        flat = routing.perm[lo:hi]
        tok = flat // k
        slot = flat % k
        # each expert is dequantised, used once and dropped, so a full-size
        # layer never holds more than one expanded expert
        Wg, Wu, Wd = _ExpertCache(layer.routed, group)(e)
        Y = swiglu_mlp(xf[tok], Wg, Wu, Wd)
        y[tok] += routing.weights[tok, slot][:, None] * Y
    if layer.shared is not None:
        Wg, Wu, Wd = _ExpertCache(layer.shared, group)(0)
        y += swiglu_mlp(xf, Wg, Wu, Wd)
    return y


def forward_dense(x, layer, routing: Routing, group: int,
                  rows: Optional[Sequence[int]] = None, cache: Optional[dict] = None) -> np.ndarray:
    """Per-token form: y_t = sum_j w[t,j] * MLP_{ids[t,j]}(x_t) + MLP_shared(x_t).

    ``rows`` restricts the computation to a subset of tokens (sampled checks).
    ``cache`` may hold dequantised experts across calls on the same layer.
    """
    xf = bf16_to_f64(x)
    T, H = xf.shape
    rows = list(range(T)) if rows is None else list(rows)
    routed = _ExpertCache(layer.routed, group)
    if cache is not None:
        routed.cache = cache.setdefault("routed", {})
    shared = None
    if layer.shared is not None:
        shared = _ExpertCache(layer.shared, group)
        if cache is not None:
            shared.cache = cache.setdefault("shared", {})
    y = np.zeros((len(rows), H), dtype=np.float64)
    for i, t in enumerate(rows):
        xt = xf[t:t + 1]
        for j in range(routing.ids.shape[1]):
            Wg, Wu, Wd = routed(int(routing.ids[t, j]))
            y[i] += routing.weights[t, j] * swiglu_mlp(xt, Wg, Wu, Wd)[0]
        if shared is not None:
            Wg, Wu, Wd = shared(0)
            y[i] += swiglu_mlp(xt, Wg, Wu, Wd)[0]
    return y


# ----------------------------------------------------------------------------
# test-input conditioning
# ----------------------------------------------------------------------------

def gap_conditioned_x(draw, T: int, router_w, router_b, top_k: int,
                      min_gap: float = 1e-3, max_attempts: int = 64):
    """Redraw rows whose k-th/(k+1)-th logit gap is below ``min_gap``.

    ``draw(redraws)`` returns x [T, H] (bf16) given {row: attempt}.  Routing ids are
    unique and identical between fp32 and fp64 logits only with a clear gap at the
    selection boundary, so the parity inputs are conditioned this way.  Returns
    (x, redraws).
    """
    redraws = {}
    for _ in range(max_attempts):
        x = draw(redraws)
        gaps = kth_gap(router_logits(x, router_w, router_b), top_k)
        bad = np.nonzero(gaps < min_gap)[0]
        if bad.size == 0:
            return x, redraws
        for t in bad:
            redraws[int(t)] = redraws.get(int(t), 0) + 1
    raise RuntimeError("could not condition the router gap")


def relative_error(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 when both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
