"""Planted mistakes: the oracle's pins must catch plausible slips.

Each case replaces one function of the CPU oracle, inside this test only, with a
version holding one plausible mistake (nibble order, a zero-point subtraction, a
wrong sign, ties to the higher index, a missing renormalisation, ids in logit
order, a reversed segment order, a swapped gate/up, a dropped routing weight, a
dropped shared expert, an ignored router bias, a bias that steers only the
choice, a sampled dense row taken from the wrong token) and runs the pins of
test_oracle.py against it: at least one pin must fail.  The oracle itself is
never modified.
"""
import dataclasses

import numpy as np
import pytest

from oracle import moe_w4_oracle as O
import test_oracle as P

_orig = {name: getattr(O, name) for name in
         ("unpack_codes", "dequant", "select_experts", "group_by_expert", "silu", "swiglu_mlp",
          "forward_grouped", "forward_dense", "router_logits", "route")}


def _pins():
    """Every pin of test_oracle.py as a zero-argument callable (parametrised ones with
    representative arguments)."""
    pins = [(f"dequant_hand_worked[{c['name']}]", lambda c=c: P.test_dequant_hand_worked_groups(c))
            for c in P._golden_cases()[1]]
    pins += [(f.__name__, f) for f in (
        P.test_dequant_is_exact_in_fp32_for_generated_data,
        P.test_logits_exact_on_integer_valued_inputs,
        P.test_topk_all_experts_is_full_softmax,
        P.test_topk_single_expert_has_weight_one_and_is_argmax,
        P.test_topk_shift_invariance_and_unit_sum,
        P.test_topk_ties_go_to_lower_index,
        P.test_router_bias_changes_selection,
        P.test_router_bias_enters_the_weights,
        P.test_grouping_matches_brute_force_counting_sort,
        P.test_single_expert_top1_no_shared_is_textbook_swiglu,
        P.test_block_matches_textbook_mixture,
        P.test_dense_rows_subset_equals_grouped_rows,
        P.test_zero_routed_weights_leave_only_shared,
        P.test_zero_input_gives_zero_output,
        P.test_duplicate_rows_route_and_output_identically,
        P.test_token_permutation_invariance,
        P.test_silu_closed_forms,
    )]
    pins += [("topk_brute_force[6,2]", lambda: P.test_topk_matches_brute_force(6, 2)),
             ("topk_brute_force[7,4]", lambda: P.test_topk_matches_brute_force(7, 4)),
             ("grouped_equals_dense", lambda: P.test_grouped_equals_dense(True))]
    return pins


def _failing_pins():
    failed = []
    for name, pin in _pins():
        try:
            pin()
        except Exception:           # an assertion, or the slip breaking a shape
            failed.append(name)
    return failed


# --- the slips -----------------------------------------------------------------

def _unpack_swapped_nibbles(packed):
    p = O._as_numpy(packed)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p >> 4          # even k taken from the high nibble
    out[..., 1::2] = p & 0x0F
    return out


def _dequant_zero_point(codes, scales, biases, group):
    return _orig["dequant"](codes, scales, biases, group) - 8.0 * _scale_per_k(scales, group)


def _scale_per_k(scales, group):
    s = O.bf16_to_f64(scales)
    return np.repeat(s, group, axis=-1)


def _dequant_bias_subtracted(codes, scales, biases, group):
    c = O.unpack_codes(codes).astype(np.float64)
    s, b = O.bf16_to_f64(scales), O.bf16_to_f64(biases)
    g = np.arange(c.shape[-1]) // group
    return c * s[..., g] - b[..., g]


def _select(logits, top_k, tie_high=False, renorm=True, ascending=True):
    T, E = logits.shape
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    for t in range(T):
        l = logits[t]
        p = np.exp(l - l.max())
        p = p / p.sum()
        order = sorted(range(E), key=lambda e: (-l[e], -e if tie_high else e))
        chosen = sorted(order[:top_k]) if ascending else order[:top_k]
        ids[t] = chosen
        w[t] = p[chosen] / (p[chosen].sum() if renorm else 1.0)
    return ids, w


def _group_reversed_segments(ids, num_experts):
    counts, offsets, perm = _orig["group_by_expert"](ids, num_experts)
    perm = perm.copy()
    for e in range(num_experts):
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    return counts, offsets, perm


def _silu_wrong_sign(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _swiglu_gate_up_swapped(X, Wg, Wu, Wd):
    return ((X @ Wg.T) * O.silu(X @ Wu.T)) @ Wd.T


def _forward_without_weights(x, layer, routing, group):
    ones = dataclasses.replace(routing, weights=np.ones_like(routing.weights))
    return _orig["forward_grouped"](x, layer, ones, group)


def _forward_without_shared(x, layer, routing, group):
    return _orig["forward_grouped"](x, dataclasses.replace(layer, shared=None), routing, group)


def _logits_without_bias(x, router_w, router_b=None):
    return _orig["router_logits"](x, router_w, None)


def _route_bias_selects_only(x, router_w, router_b, top_k):
    """The bias steers the choice, but the weights come from the raw logits."""
    biased = _orig["route"](x, router_w, router_b, top_k)
    if router_b is None:
        return biased
    raw = _orig["router_logits"](x, router_w, None)
    w = np.empty_like(biased.weights)
    for t in range(raw.shape[0]):
        p = np.exp(raw[t] - raw[t].max())
        w[t] = p[biased.ids[t]] / p[biased.ids[t]].sum()
    return dataclasses.replace(biased, weights=w)


def _dense_rows_misindexed(x, layer, routing, group, rows=None, cache=None):
    """Output row i computed from token i instead of token rows[i]."""
    if rows is None:
        return _orig["forward_dense"](x, layer, routing, group, cache=cache)
    rows = list(rows)
    full = _orig["forward_dense"](x, layer, routing, group, cache=cache)
    return full[list(range(len(rows)))]


SLIPS = {
    "nibble order swapped": ("unpack_codes", _unpack_swapped_nibbles),
    "zero point 8 subtracted": ("dequant", _dequant_zero_point),
    "bias subtracted": ("dequant", _dequant_bias_subtracted),
    "ties to the higher index": ("select_experts", lambda l, k: _select(l, k, tie_high=True)),
    "no renormalisation": ("select_experts", lambda l, k: _select(l, k, renorm=False)),
    "ids in logit order": ("select_experts", lambda l, k: _select(l, k, ascending=False)),
    "segments in reverse token order": ("group_by_expert", _group_reversed_segments),
    "silu sign": ("silu", _silu_wrong_sign),
    "gate and up swapped": ("swiglu_mlp", _swiglu_gate_up_swapped),
    "routing weight dropped": ("forward_grouped", _forward_without_weights),
    "shared expert dropped": ("forward_grouped", _forward_without_shared),
    "router bias ignored": ("router_logits", _logits_without_bias),
    "router bias used for selection only": ("route", _route_bias_selects_only),
    "dense rows misindexed": ("forward_dense", _dense_rows_misindexed),
}


def test_pins_pass_on_the_oracle():
    assert _failing_pins() == []


@pytest.mark.parametrize("slip", sorted(SLIPS))
def test_pins_catch_planted_slip(slip, monkeypatch):
    name, fn = SLIPS[slip]
    monkeypatch.setattr(O, name, fn)
    failed = _failing_pins()
    print(f"{slip}: caught by {failed}")
    assert failed, f"no pin catches: {slip}"
