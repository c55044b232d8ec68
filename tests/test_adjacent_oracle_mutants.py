"""Planted mistakes in the decode-attention and Gated DeltaNet oracles.

As for the MoE oracle: each case replaces the oracle's function, inside this test
only, with a version holding one plausible slip, runs the pins of
test_attn_oracle.py / test_gdn_oracle.py against it, and requires at least one pin
to fail.  The oracles themselves are never modified.
"""
import math

import numpy as np
import pytest

from oracle import attn_oracle as A
from oracle import gdn_oracle as G
import test_attn_oracle as PA
import test_gdn_oracle as PG

_attn = A.decode_attention
_gather = A.gather_cache
_scan = G.gdn_scan


def _run(pins):
    failed = []
    for name, pin in pins:
        try:
            pin()
        except Exception:           # an assertion, or the slip breaking a shape
            failed.append(name)
    return failed


def _attn_pins():
    pins = [(f.__name__, f) for f in (
        PA.test_one_token_context_returns_its_value, PA.test_identical_keys_give_the_mean_value,
        PA.test_dominant_key_returns_its_value_row, PA.test_brute_force_python_loops,
        PA.test_block_table_permutation_invariance, PA.test_shift_invariance_of_the_scores,
        PA.test_output_in_convex_hull_of_values, PA.test_poisoned_tail_is_not_read,
        PA.test_large_scores_stay_finite)]
    pins += [(f"gqa[{hq},{hkv}]", lambda hq=hq, hkv=hkv: PA.test_gqa_mapping_matches_repeated_cache_heads(hq, hkv))
             for hq, hkv in ((16, 2), (8, 2))]
    return pins


def _gdn_pins():
    pins = [(f.__name__, f) for f in (
        PG.test_beta_zero_is_pure_decay, PG.test_exact_recall_of_orthonormal_keys,
        PG.test_repeated_key_is_overwritten, PG.test_matches_the_product_form_with_explicit_matrices,
        PG.test_linear_in_initial_state_and_values, PG.test_split_sequence_with_state_carried_over,
        PG.test_q_and_k_play_different_roles)]
    pins += [(f"heads[{hv},{hk}]", lambda hv=hv, hk=hk: PG.test_head_mapping_matches_repeated_heads(hv, hk))
             for hv, hk in ((4, 2), (6, 3))]
    return pins


# --- decode attention slips ------------------------------------------------------

def _attention(q, k_pool, v_pool, table, n_ctx, scale=None, *, interleaved=False, scale_1_over_d=False,
               no_max=False, drop_newest=False):
    Q = A._f64(q)
    Hq, d = Q.shape
    Kd, Vd = A.gather_cache(k_pool, v_pool, table, n_ctx - 1 if drop_newest else n_ctx)
    Hkv = Kd.shape[0]
    Gq = Hq // Hkv
    if scale is None:
        scale = 1.0 / d if scale_1_over_d else 1.0 / math.sqrt(d)
    out = np.empty((Hq, d), dtype=np.float64)
    for h in range(Hq):
        c = h % Hkv if interleaved else h // Gq
        s = (Kd[c] @ Q[h]) * scale
        if not no_max:
            s = s - s.max()
        with np.errstate(over="ignore", invalid="ignore"):
            p = np.exp(s)
            p = p / p.sum()
        out[h] = p @ Vd[c]
    return out


def _gather_ignoring_table(k_pool, v_pool, table, n_ctx):
    K, V = A._f64(k_pool), A._f64(v_pool)
    B = K.shape[2]
    n = np.arange(n_ctx)
    return K[n // B, :, n % B, :].transpose(1, 0, 2), V[n // B, :, n % B, :].transpose(1, 0, 2)


ATTN_SLIPS = {
    "query heads interleaved over cache heads": ("decode_attention", lambda *a, **kw: _attention(*a, interleaved=True, **kw)),
    "scale 1/d": ("decode_attention", lambda *a, **kw: _attention(*a, scale_1_over_d=True, **kw)),
    "no max subtraction": ("decode_attention", lambda *a, **kw: _attention(*a, no_max=True, **kw)),
    "newest token dropped": ("decode_attention", lambda *a, **kw: _attention(*a, drop_newest=True, **kw)),
    "block table ignored": ("gather_cache", _gather_ignoring_table),
}


# --- Gated DeltaNet slips ----------------------------------------------------------

def _gdn(q, k, v, g, beta, state, *, decay_after=False, no_decay_in_delta=False, out_with_k=False,
         heads_interleaved=False, out_before_update=False, no_beta=False):
    Q, K, V = G._f64(q), G._f64(k), G._f64(v)
    Gd, Bt = G._f64(g), G._f64(beta)
    S = G._f64(state).copy()
    T, Hk, d = Q.shape
    Hv = V.shape[1]
    rep = Hv // Hk
    head_of = (np.arange(Hv) % Hk) if heads_interleaved else (np.arange(Hv) // rep)
    out = np.empty((T, Hv, d), dtype=np.float64)
    for t in range(T):
        kt, qt = K[t, head_of], Q[t, head_of]
        a = np.exp(Gd[t])[:, None, None]
        b = np.ones((Hv, 1)) if no_beta else Bt[t][:, None]
        if out_before_update:
            out[t] = np.einsum("hij,hj->hi", S, kt if out_with_k else qt)
        Sk = np.einsum("hij,hj->hi", S, kt)
        if decay_after:
            S = a * (S + (b * (V[t] - Sk))[:, :, None] * kt[:, None, :])
        else:
            delta = b * (V[t] - (Sk if no_decay_in_delta else a[:, :, 0] * Sk))
            S = a * S + delta[:, :, None] * kt[:, None, :]
        if not out_before_update:
            out[t] = np.einsum("hij,hj->hi", S, kt if out_with_k else qt)
    return out, S


GDN_SLIPS = {
    "decay applied after the write": dict(decay_after=True),
    "decay missing from the correction": dict(no_decay_in_delta=True),
    "output read with k instead of q": dict(out_with_k=True),
    "value heads interleaved over key heads": dict(heads_interleaved=True),
    "output read before the update": dict(out_before_update=True),
    "write strength ignored": dict(no_beta=True),
}


def test_pins_pass_on_the_adjacent_oracles():
    assert _run(_attn_pins()) == []
    assert _run(_gdn_pins()) == []


@pytest.mark.parametrize("slip", sorted(ATTN_SLIPS))
def test_attention_pins_catch_planted_slip(slip, monkeypatch):
    name, fn = ATTN_SLIPS[slip]
    monkeypatch.setattr(A, name, fn)
    failed = _run(_attn_pins())
    print(f"{slip}: caught by {failed}")
    assert failed, f"no pin catches: {slip}"


@pytest.mark.parametrize("slip", sorted(GDN_SLIPS))
def test_gdn_pins_catch_planted_slip(slip, monkeypatch):
    kw = GDN_SLIPS[slip]
    monkeypatch.setattr(G, "gdn_scan", lambda *a: _gdn(*a, **kw))
    failed = _run(_gdn_pins())
    print(f"{slip}: caught by {failed}")
    assert failed, f"no pin catches: {slip}"
