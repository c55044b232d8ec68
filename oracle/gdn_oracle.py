"""CPU oracle for the Gated DeltaNet scan.  TEST INFRASTRUCTURE ONLY.

Only the test-suite and the benchmark's CPU-baseline leg may import this module.
It shares no code with the HIP path; its only shared dependency is the seeded
input generator (``w4_dequant_grouped_amd/synth_gdn.py``).

The pages name the operation and nothing more: 30 of the model's 40 layers run
Gated DeltaNet with a recurrent state of fixed size ("Perplexity built an
inference engine for one model, one chip", paragraph 2), and a register-resident
scan of it sped up prefill ("Perplexity's Lily brings fast local AI to Apple
silicon Macs", section "Where the Engine Gains Speed").  The recurrence is the
published gated delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta Networks:
Improving Mamba2 with Delta Rule", ICLR 2025), per value head h with query/key
head c = h // (Hv / Hk), state S (value rows x key columns), for t = 1 .. T:

    alpha_t = exp(g_t)
    S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T
    o_t = S_t q_t

i.e. decay the state, then move its value at key k_t a fraction beta_t of the way
to v_t.  The oracle runs it token by token in float64 (vectorised over heads and
value rows only) and returns the outputs and the final state.

Readings where the pages are silent: the recurrence above (its published form);
q and k arrive normalised (the scan does not normalise or scale them); g is the
log-decay and beta the write strength, one each per value head and token; the
state is carried in and out in fp32.

Pinned by tests/test_gdn_oracle.py: beta = 0 (pure decay, closed form), exact
recall of orthonormal keys with alpha = beta = 1, overwrite of a repeated key, the
paper's product form S_{t-1} (alpha (I - beta k k^T)) + beta v k^T computed with
explicit matrices, linearity, splitting the sequence with the state carried over,
and the head mapping against repeated query/key heads.
"""
from __future__ import annotations

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _f64(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def gdn_scan(q, k, v, g, beta, state):
    """Outputs o [T][Hv][d] and the final state [Hv][d][d], float64."""
    Q, K, V = _f64(q), _f64(k), _f64(v)
    G, Bt = _f64(g), _f64(beta)
    S = _f64(state).copy()
    T, Hk, d = Q.shape
    Hv = V.shape[1]
    assert Hv % Hk == 0
    rep = Hv // Hk
    head_of = np.arange(Hv) // rep             # query/key head of each value head
    out = np.empty((T, Hv, d), dtype=np.float64)
    for t in range(T):
        kt = K[t, head_of]                     # [Hv][d]
        qt = Q[t, head_of]
        a = np.exp(G[t])[:, None, None]        # [Hv][1][1]
        b = Bt[t][:, None]                     # [Hv][1]
        Sk = np.einsum("hij,hj->hi", S, kt)    # S_{t-1} k_t, [Hv][d]
        delta = b * (V[t] - a[:, :, 0] * Sk)   # beta (v - alpha S k)
        S = a * S + delta[:, :, None] * kt[:, None, :]
        out[t] = np.einsum("hij,hj->hi", S, qt)
    return out, S


def relative_error(got, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
