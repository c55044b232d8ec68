"""Pins for the CPU oracle: each checks it against something other than itself.

Hand-worked dequantisation groups, exact integer-valued router logits, brute
force over expert subsets, a brute-force counting sort, the textbook SwiGLU MLP
written with torch's own functions, closed-form special cases and invariances.
A plausible slip anywhere in the oracle (nibble order, group index, a swapped
gate/up, a missing renormalisation, a misaligned weight, a wrong scatter row, a
dropped shared expert) fails at least one of these.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import moe_w4_oracle as O
from w4_dequant_grouped_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dequant_groups.json")


def _bits_to_bf16(rows):
    arr = np.array([[int(b, 16) for b in r] for r in rows], dtype=np.uint16)
    return arr


# ---------------------------------------------------------------------------
# dequantisation
# ---------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        doc = json.load(f)
    assert "A 35B Model Built for Local Memory" in doc["citation"]
    return doc["group"], doc["cases"]


@pytest.mark.parametrize("case", _golden_cases()[1], ids=lambda c: c["name"])
def test_dequant_hand_worked_groups(case):
    group = _golden_cases()[0]
    N, K = case["N"], case["K"]
    if "packed_hex_rows" in case:
        rows = [bytes.fromhex(h) for h in case["packed_hex_rows"]]
    else:
        rows = [bytes.fromhex(case["packed_hex_row_period"] * case["packed_period_repeat"])]
    codes = np.frombuffer(b"".join(rows), dtype=np.uint8).reshape(N, K // 2)
    scales = _bits_to_bf16(case["scale_bits"])
    biases = _bits_to_bf16(case["bias_bits"])
    got = O.dequant(codes, scales, biases, group)
    if "expected_rows_const" in case:
        want = [[Fraction(v)] * K for v in case["expected_rows_const"]]
    else:
        # expected_period[g] lists the values of group g, repeated to fill the group
        row = []
        for vals in case["expected_period"]:
            row += [Fraction(v) for v in vals] * case["expected_period_repeat"]
        want = [row] * N
    assert got.shape == (N, K)
    for n in range(N):
        for k in range(K):
            assert Fraction(got[n, k]) == want[n][k], (case["name"], n, k, got[n, k], want[n][k])


def test_dequant_is_exact_in_fp32_for_generated_data():
    # code*scale has <= 12 significant bits and adding the bf16 bias stays within
    # float32's 24, so dequantising in float32 equals the float64 value exactly.
    gen = synth.generator(5)
    m = synth.draw_w4(gen, 2, 8, 256)
    w64 = O.dequant(m.codes, m.scales, m.biases, 64)
    c = O.unpack_codes(m.codes).astype(np.float32)
    s = m.scales.float().numpy()[..., np.arange(256) // 64]
    b = m.biases.float().numpy()[..., np.arange(256) // 64]
    w32 = c * s + b
    assert np.array_equal(w32.astype(np.float64), w64)


# ---------------------------------------------------------------------------
# router logits / selection
# ---------------------------------------------------------------------------

def test_logits_exact_on_integer_valued_inputs():
    rng = np.random.default_rng(1)
    T, H, E = 5, 96, 7
    x_int = rng.integers(-1, 2, size=(T, H))
    wr_num = rng.integers(-512, 513, size=(E, H))            # W_r = num / 1024
    b_num = rng.integers(-4096, 4097, size=E)                # b_r = num / 1024
    x = torch.tensor(x_int, dtype=torch.float32).to(torch.bfloat16)
    wr = torch.tensor(wr_num / 1024.0, dtype=torch.float32)
    br = torch.tensor(b_num / 1024.0, dtype=torch.float32)
    got = O.router_logits(x, wr, br)
    for t in range(T):
        for e in range(E):
            exact = Fraction(int(sum(int(x_int[t, h]) * int(wr_num[e, h]) for h in range(H)))
                             + int(b_num[e]), 1024)
            assert Fraction(got[t, e]) == exact


def _brute_topk(l, k):
    """Best k-subset by total logit (unique for distinct logits) and exp-ratio weights."""
    E = len(l)
    best = max(itertools.combinations(range(E), k), key=lambda S: sum(l[i] for i in S))
    den = sum(math.exp(l[i]) for i in best)
    return list(best), [math.exp(l[i]) / den for i in best]


@pytest.mark.parametrize("E,k", [(6, 1), (6, 2), (6, 3), (7, 4), (5, 5)])
def test_topk_matches_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    logits = rng.normal(size=(9, E)) * 2.0
    ids, w = O.select_experts(logits, k)
    for t in range(logits.shape[0]):
        bids, bw = _brute_topk(list(logits[t]), k)
        assert list(ids[t]) == bids
        np.testing.assert_allclose(w[t], bw, rtol=1e-13, atol=0)


def test_topk_all_experts_is_full_softmax():
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    logits = rng.normal(size=(4, 9)) * 3
    ids, w = O.select_experts(logits, 9)
    assert (ids == np.arange(9)).all()
    np.testing.assert_allclose(w, softmax(logits, axis=1), rtol=1e-13)


def test_topk_single_expert_has_weight_one_and_is_argmax():
    rng = np.random.default_rng(4)
    logits = rng.normal(size=(20, 11))
    ids, w = O.select_experts(logits, 1)
    assert (ids[:, 0] == logits.argmax(axis=1)).all()
    assert (w == 1.0).all()


def test_topk_shift_invariance_and_unit_sum():
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(12, 16))
    ids, w = O.select_experts(logits, 4)
    ids2, w2 = O.select_experts(logits + 37.25, 4)
    assert (ids == ids2).all()
    np.testing.assert_allclose(w, w2, rtol=1e-12)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (np.diff(ids, axis=1) > 0).all()   # ascending expert ids


def test_topk_ties_go_to_lower_index():
    logits = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    ids, w = O.select_experts(logits, 2)
    assert list(ids[0]) == [1, 2]
    np.testing.assert_allclose(w[0], [0.5, 0.5])


def test_router_bias_changes_selection():
    x = torch.ones((1, 64), dtype=torch.bfloat16)
    wr = torch.zeros((4, 64), dtype=torch.float32)
    wr[0] = 1.0 / 64     # logit 1 without bias
    br = torch.tensor([0.0, 0.0, 0.0, 5.0])
    r = O.route(x, wr, br, 1)
    assert r.ids[0, 0] == 3
    r0 = O.route(x, wr, None, 1)
    assert r0.ids[0, 0] == 0


def test_router_bias_enters_the_weights():
    """Hand-worked top-2 of three experts with a router bias.  x is all ones over
    64 hidden units and W_r's rows are constant, so the raw logits are exactly
    (1, 2, 0); the bias (0, -1.5, 2) makes them (1, 0.5, 2).  The biased logits
    choose experts 0 and 2 (the raw ones would choose 0 and 1), and the weights
    are the softmax of the biased chosen logits: 1/(1+e) and e/(1+e).  A bias
    that steered only the choice would give the softmax of the raw logits
    (1, 0) instead: e/(1+e) and 1/(1+e), the two weights swapped."""
    x = torch.ones((1, 64), dtype=torch.bfloat16)
    wr = torch.zeros((3, 64), dtype=torch.float32)
    wr[0] = 1.0 / 64
    wr[1] = 2.0 / 64
    br = torch.tensor([0.0, -1.5, 2.0])
    r = O.route(x, wr, br, 2)
    assert list(r.logits[0]) == [1.0, 0.5, 2.0]
    assert list(r.ids[0]) == [0, 2]
    e = math.e
    np.testing.assert_allclose(r.weights[0], [1.0 / (1.0 + e), e / (1.0 + e)], rtol=1e-14, atol=0)
    r0 = O.route(x, wr, None, 2)
    assert list(r0.ids[0]) == [0, 1]
    np.testing.assert_allclose(r0.weights[0], [1.0 / (1.0 + e), e / (1.0 + e)], rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# grouping
# ---------------------------------------------------------------------------

def test_grouping_matches_brute_force_counting_sort():
    rng = np.random.default_rng(6)
    T, E, k = 37, 10, 3
    ids = np.sort(np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]), axis=1)
    counts, offsets, perm = O.group_by_expert(ids.astype(np.int32), E)
    want_perm = []
    for e in range(E):
        for t in range(T):
            for s in range(k):
                if ids[t, s] == e:
                    want_perm.append(t * k + s)
    want_counts = [sum(int((ids[t] == e).any()) for t in range(T)) for e in range(E)]
    assert list(counts) == want_counts
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert list(np.diff(offsets)) == want_counts
    assert list(perm) == want_perm
    assert sorted(perm) == list(range(T * k))


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------

def _tiny_layer(seed, T=6, H=128, I=64, E=5, k=2, shared=True, bias=False):
    shape = synth.BlockShape(T=T, H=H, I=I, E=E, top_k=k, shared=shared,
                             router_bias="zipf" if bias else "none")
    layer = synth.draw_layer(shape, seed)
    x = synth.draw_x(T, H, seed)
    return shape, layer, x


def _torch_swiglu(x, wg, wu, wd):
    """Textbook SwiGLU MLP with torch's own ops, float64."""
    x, wg, wu, wd = (torch.from_numpy(a) for a in (x, wg, wu, wd))
    h = torch.nn.functional.silu(torch.nn.functional.linear(x, wg)) * torch.nn.functional.linear(x, wu)
    return torch.nn.functional.linear(h, wd).numpy()


def test_single_expert_top1_no_shared_is_textbook_swiglu():
    shape, layer, x = _tiny_layer(7, T=5, H=128, I=64, E=1, k=1, shared=False)
    r = O.route(x, layer.router_w, None, 1)
    y = O.forward_grouped(x, layer, r, 64)
    m = layer.routed
    wg = O.dequant(m.gate.codes[0], m.gate.scales[0], m.gate.biases[0], 64)
    wu = O.dequant(m.up.codes[0], m.up.scales[0], m.up.biases[0], 64)
    wd = O.dequant(m.down.codes[0], m.down.scales[0], m.down.biases[0], 64)
    ref = _torch_swiglu(O.bf16_to_f64(x), wg, wu, wd)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_block_matches_textbook_mixture():
    """Brute-force routing + torch SwiGLU per expert, weighted sum + shared."""
    shape, layer, x = _tiny_layer(8, T=7, H=128, I=64, E=5, k=2, shared=True)
    r = O.route(x, layer.router_w, None, 2)
    xf = O.bf16_to_f64(x)
    l = xf @ layer.router_w.double().numpy().T
    m, sh = layer.routed, layer.shared

    def mats(ex, e):
        return [O.dequant(getattr(ex, n).codes[e], getattr(ex, n).scales[e],
                          getattr(ex, n).biases[e], 64) for n in ("gate", "up", "down")]

    ref = np.zeros_like(xf)
    for t in range(shape.T):
        bids, bw = _brute_topk(list(l[t]), 2)
        for e, w in zip(bids, bw):
            ref[t] += w * _torch_swiglu(xf[t:t + 1], *mats(m, e))[0]
        ref[t] += _torch_swiglu(xf[t:t + 1], *mats(sh, 0))[0]
    y = O.forward_grouped(x, layer, r, 64)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("bias", [False, True])
def test_grouped_equals_dense(bias):
    shape, layer, x = _tiny_layer(9, T=19, H=128, I=64, E=8, k=3, bias=bias)
    r = O.route(x, layer.router_w, layer.router_b, 3)
    yg = O.forward_grouped(x, layer, r, 64)
    yd = O.forward_dense(x, layer, r, 64)
    assert O.relative_error(yg, yd) <= 1e-12


def test_dense_rows_subset_equals_grouped_rows():
    """forward_dense over a subset of tokens, in the caller's (unsorted) order and
    with a shared dequantisation cache across two calls, returns exactly those rows
    of the grouped form: the sampled full-size parity checks rest on this."""
    shape, layer, x = _tiny_layer(14, T=23, H=128, I=64, E=8, k=3, bias=True)
    r = O.route(x, layer.router_w, layer.router_b, 3)
    yg = O.forward_grouped(x, layer, r, 64)
    rows = [17, 0, 22, 5, 9]
    cache = {}
    yd = O.forward_dense(x, layer, r, 64, rows=rows, cache=cache)
    assert yd.shape == (len(rows), shape.H)
    assert O.relative_error(yd, yg[rows]) <= 1e-12
    yd2 = O.forward_dense(x, layer, r, 64, rows=[3, 17], cache=cache)
    assert O.relative_error(yd2, yg[[3, 17]]) <= 1e-12


def test_zero_routed_weights_leave_only_shared():
    shape, layer, x = _tiny_layer(10, T=4, H=128, I=64, E=4, k=2)
    for mat in (layer.routed.gate, layer.routed.up, layer.routed.down):
        mat.codes[:] = 0x88                             # every code 8
        mat.biases.copy_((-8.0 * mat.scales.float()).to(torch.bfloat16))  # exact: 8s fits bf16
    r = O.route(x, layer.router_w, None, 2)
    y = O.forward_grouped(x, layer, r, 64)
    sh = layer.shared
    mats = [O.dequant(getattr(sh, n).codes[0], getattr(sh, n).scales[0], getattr(sh, n).biases[0], 64)
            for n in ("gate", "up", "down")]
    ref = _torch_swiglu(O.bf16_to_f64(x), *mats)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_zero_input_gives_zero_output():
    shape, layer, _ = _tiny_layer(11)
    x = torch.zeros((shape.T, shape.H), dtype=torch.bfloat16)
    r = O.route(x, layer.router_w, None, shape.top_k)
    assert (O.forward_grouped(x, layer, r, 64) == 0).all()


def test_duplicate_rows_route_and_output_identically():
    shape, layer, x = _tiny_layer(12, T=6)
    x[3] = x[1]
    r = O.route(x, layer.router_w, None, shape.top_k)
    y = O.forward_grouped(x, layer, r, 64)
    assert (r.ids[3] == r.ids[1]).all()
    assert np.array_equal(y[3], y[1])


def test_token_permutation_invariance():
    shape, layer, x = _tiny_layer(13, T=11, E=6, k=2)
    p = torch.randperm(shape.T, generator=synth.generator(99))
    r = O.route(x, layer.router_w, None, 2)
    rp = O.route(x[p], layer.router_w, None, 2)
    y = O.forward_grouped(x, layer, r, 64)
    yp = O.forward_grouped(x[p], layer, rp, 64)
    pn = p.numpy()
    assert (rp.ids == r.ids[pn]).all()
    np.testing.assert_allclose(rp.weights, r.weights[pn], rtol=1e-14)
    assert (rp.counts == r.counts).all() and (rp.offsets == r.offsets).all()
    np.testing.assert_allclose(yp, y[pn], rtol=1e-12, atol=1e-13)
    # perm relabelled: entry (t*k+s) of the permuted batch is row p[t] of the original
    inv = {int(pn[t]) * 2 + s: t * 2 + s for t in range(shape.T) for s in range(2)}
    for e in range(6):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        relabelled = sorted(inv[int(v)] for v in r.perm[lo:hi])
        assert list(rp.perm[lo:hi]) == relabelled


def test_silu_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -800.0])
    got = O.silu(z)
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(got[2] - (-0.25 * math.log(3.0))) < 1e-15
    assert abs(got[3] - 40.0) < 1e-12
    assert got[4] == 0.0


def test_gap_conditioning_enforces_the_gap():
    shape = synth.BlockShape(T=64, H=256, I=64, E=16, top_k=4)
    layer = synth.draw_layer(shape, 21)
    x, redraws = O.gap_conditioned_x(
        lambda rd: synth.draw_x(shape.T, shape.H, 21, redraws=rd),
        shape.T, layer.router_w, None, 4, min_gap=0.05)
    gaps = O.kth_gap(O.router_logits(x, layer.router_w, None), 4)
    assert gaps.min() >= 0.05
    assert len(redraws) > 0        # with a 0.05 floor some rows must be redrawn


def test_relative_error_metric():
    assert O.relative_error(np.array([1.0, 2.0]), np.array([1.0, 2.0])) == 0.0
    assert O.relative_error(np.array([1.0, 2.5]), np.array([1.0, 2.0])) == 0.25
    assert O.relative_error(np.zeros(3), np.zeros(3)) == 0.0


def test_zipf_router_bias_skews_loads_at_2048_tokens():
    """The skewed prefill workload must have experts above 4x the mean load and empty ones."""
    wl = synth.WORKLOADS["prefill2048_zipf"]
    sh = wl.shape
    wr, br = synth.draw_router(sh, wl.seed)
    x = synth.draw_x(sh.T, sh.H, wl.seed)
    logits = O.router_logits(x, wr, br)
    top = np.argsort(-logits, axis=1)[:, :sh.top_k]
    loads = np.bincount(top.ravel(), minlength=sh.E)
    mean = sh.T * sh.top_k / sh.E
    assert (loads > 4 * mean).sum() >= 5
    assert (loads == 0).sum() >= 1
    # without the bias the same tokens spread evenly
    flat = np.bincount(np.argsort(-O.router_logits(x, wr, None), axis=1)[:, :sh.top_k].ravel(),
                       minlength=sh.E)
    assert flat.max() < 2 * mean and (flat == 0).sum() == 0


def test_draw_router_matches_draw_layer():
    sh = synth.BlockShape(T=4, H=128, I=64, E=8, top_k=2, router_bias="zipf")
    wr, br = synth.draw_router(sh, 31)
    layer = synth.draw_layer(sh, 31)
    assert torch.equal(wr, layer.router_w) and torch.equal(br, layer.router_b)
