"""CPU oracle for one decode-attention step over a paged KV cache.
TEST INFRASTRUCTURE ONLY.

Only the test-suite and the benchmark's CPU-baseline leg may import this module.
It shares no code with the HIP path; its only shared dependency is the seeded
input generator (``w4_dequant_grouped_amd/synth_attn.py``).

What it computes is the plain definition of scaled dot-product attention for one
query token, written out in float64 with NumPy:

  for query head h, with key/value head c = h // (Hq / Hkv):
      s_n = (q_h . k_{c,n}) / sqrt(d)            for every cached token n < n_ctx
      p_n = exp(s_n - max_m s_m) / sum_m exp(s_m - max_m s_m)
      o_h = sum_n p_n v_{c,n}

The pages name the head layout (16 query heads over two key/value heads: "Perplexity's
Lily brings fast local AI to Apple silicon Macs", section "A 35B Model Built for
Local Memory") and say that the engine packs the query heads of a group so that a
cached key/value row is read once and lays the cache out in fixed-size blocks
("Perplexity built an inference engine for one model, one chip", paragraph 3;
"Perplexity's Lily ...", section "Where the Engine Gains Speed").  Packing and the
block layout change how the cache is read, not the result, so the oracle is the
unpacked definition; the block table is only used to find token n's row.

Readings where the pages are silent: query head h uses key/value head
h // (Hq / Hkv) (consecutive query heads share a cache head); the scale is
1 / sqrt(head_dim); the cache already holds the new token's key and value; token
n sits in slot n % B of logical block n // B.  One page says four query heads are
grouped, another gives 16 query and two key/value heads; the group size here is
Hq / Hkv (8 for the model) and the tests also cover a group of 4.

Pinned by tests/test_attn_oracle.py: a one-token context, identical keys (the mean
of the values), a dominant key, brute force with Python loops, the block table's
permutation invariance, the shift invariance of softmax, the GQA head mapping and
the convex-hull bound.
"""
from __future__ import annotations

import math

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _f64(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def gather_cache(k_pool, v_pool, table, n_ctx: int):
    """Dense K, V [Hkv][n_ctx][d] (float64) read through the block table."""
    K = _f64(k_pool)
    V = _f64(v_pool)
    tab = np.asarray(table.cpu() if torch is not None and isinstance(table, torch.Tensor) else table,
                     dtype=np.int64)
    B = K.shape[2]
    n = np.arange(n_ctx)
    phys = tab[n // B]
    slot = n % B
    # K[phys, :, slot, :] has shape [n_ctx, Hkv, d]
    return K[phys, :, slot, :].transpose(1, 0, 2), V[phys, :, slot, :].transpose(1, 0, 2)


def decode_attention(q, k_pool, v_pool, table, n_ctx: int, scale: float = None) -> np.ndarray:
    """o [Hq][d] (float64) for one query token over the first n_ctx cached tokens."""
    Q = _f64(q)
    Hq, d = Q.shape
    Kd, Vd = gather_cache(k_pool, v_pool, table, n_ctx)
    Hkv = Kd.shape[0]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((Hq, d), dtype=np.float64)
    for h in range(Hq):
        c = h // G
        s = (Kd[c] @ Q[h]) * scale
        s = s - s.max()
        p = np.exp(s)
        p = p / p.sum()
        out[h] = p @ Vd[c]
    return out


def relative_error(got, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
