"""Pins for the decode-attention oracle: each checks it against something other
than itself.

A one-token context (the output is that token's value row), identical keys (the
mean of the values), a dominant key (its value row, within the softmax tail),
brute force with plain Python loops and math.exp (its own block-table lookup),
the block table's permutation invariance, softmax's shift invariance, the GQA
head mapping against repeated cache heads, and the convex-hull bound.  A slip in
the oracle (a transposed head mapping, a wrong slot or block index, a missing
scale or max subtraction, softmax over the wrong axis) fails one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attn_oracle as A
from w4_dequant_grouped_amd import synth_attn as SA


def _inputs(n_ctx, Hq=4, Hkv=2, d=8, B=4, seed=0):
    shape = SA.AttnShape(n_ctx=n_ctx, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B)
    return shape, SA.draw_attn(shape, seed)


def test_one_token_context_returns_its_value():
    shape, x = _inputs(1)
    o = A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, 1)
    phys = int(x.table[0])
    V = x.v_pool.double().numpy()
    G = shape.n_q_heads // shape.n_kv_heads
    for h in range(shape.n_q_heads):
        assert np.array_equal(o[h], V[phys, h // G, 0])


def test_identical_keys_give_the_mean_value():
    shape, x = _inputs(13, seed=1)
    k = x.k_pool.clone()
    k[:] = k[0, 0, 0]                       # every key row the same
    o = A.decode_attention(x.q, k, x.v_pool, x.table, 13)
    _, Vd = A.gather_cache(k, x.v_pool, x.table, 13)
    G = shape.n_q_heads // shape.n_kv_heads
    for h in range(shape.n_q_heads):
        np.testing.assert_allclose(o[h], Vd[h // G].mean(axis=0), rtol=0, atol=1e-12)


def test_dominant_key_returns_its_value_row():
    # key n* = 40 * q_h for the single head; the others have |s| <= ~3
    shape, x = _inputs(23, Hq=1, Hkv=1, d=8, B=4, seed=2)
    n_star = 17
    phys, slot = int(x.table[n_star // 4]), n_star % 4
    k = x.k_pool.clone()
    k[phys, 0, slot] = (40 * x.q[0].float()).to(torch.bfloat16)
    o = A.decode_attention(x.q, k, x.v_pool, x.table, 23)
    v_star = x.v_pool[phys, 0, slot].double().numpy()
    # the other 22 weights are each below exp(-(gap)), gap >= 40 |q|^2 / sqrt(8) - 10
    qn = float((x.q[0].double() ** 2).sum())
    gap = 40 * qn / math.sqrt(8) - 10
    assert gap > 30
    np.testing.assert_allclose(o[0], v_star, rtol=0, atol=22 * math.exp(-gap) * 10)


def test_brute_force_python_loops():
    shape, x = _inputs(11, Hq=4, Hkv=2, d=3, B=4, seed=3)
    q = x.q.double().tolist()
    kp = x.k_pool.double().tolist()
    vp = x.v_pool.double().tolist()
    tab = x.table.tolist()
    G = 2
    o = A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, 11)
    for h in range(4):
        c = h // G
        scores = []
        for n in range(11):
            blk, slot = divmod(n, 4)
            kr = kp[tab[blk]][c][slot]
            scores.append(sum(q[h][i] * kr[i] for i in range(3)) / math.sqrt(3))
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        z = sum(w)
        for i in range(3):
            ref = sum(w[n] * vp[tab[n // 4]][c][n % 4][i] for n in range(11)) / z
            assert abs(o[h][i] - ref) < 1e-12


def test_block_table_permutation_invariance():
    shape, x = _inputs(29, seed=4)
    P = shape.n_pool_blocks
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5))
    # move physical block b to position perm[b]
    k2 = torch.empty_like(x.k_pool)
    v2 = torch.empty_like(x.v_pool)
    k2[perm] = x.k_pool
    v2[perm] = x.v_pool
    t2 = perm[x.table.long()].to(torch.int32)
    o1 = A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, 29)
    o2 = A.decode_attention(x.q, k2, v2, t2, 29)
    assert np.array_equal(o1, o2)


def test_shift_invariance_of_the_scores():
    # adding c to every key shifts head h's scores by q_h . c / sqrt(d): same output
    shape, x = _inputs(17, Hq=2, Hkv=1, d=8, seed=6)
    K = x.k_pool.double()
    c = torch.randn(8, dtype=torch.float64, generator=torch.Generator().manual_seed(7))
    o1 = A.decode_attention(x.q, K, x.v_pool, x.table, 17)
    o2 = A.decode_attention(x.q, K + c, x.v_pool, x.table, 17)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (8, 2), (4, 4)])
def test_gqa_mapping_matches_repeated_cache_heads(Hq, Hkv):
    # query head h reads cache head h // G: repeating each cache head G times in a
    # row (one cache head per query head) must give the same output
    shape, x = _inputs(19, Hq=Hq, Hkv=Hkv, d=8, seed=8)
    G = Hq // Hkv
    o1 = A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, 19)
    o2 = A.decode_attention(x.q, x.k_pool.repeat_interleave(G, dim=1),
                            x.v_pool.repeat_interleave(G, dim=1), x.table, 19)
    assert np.array_equal(o1, o2)


def test_output_in_convex_hull_of_values():
    shape, x = _inputs(37, seed=9)
    o = A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, 37)
    _, Vd = A.gather_cache(x.k_pool, x.v_pool, x.table, 37)
    G = shape.n_q_heads // shape.n_kv_heads
    for h in range(shape.n_q_heads):
        assert (o[h] <= Vd[h // G].max(axis=0) + 1e-12).all()
        assert (o[h] >= Vd[h // G].min(axis=0) - 1e-12).all()


def test_poisoned_tail_is_not_read():
    # slots past n_ctx and unused pool blocks hold NaN: the output stays finite
    shape = SA.AttnShape(n_ctx=10, n_q_heads=4, n_kv_heads=2, head_dim=8, block=4, poison_tail=True)
    x = SA.draw_attn(shape, 10)
    assert torch.isnan(x.k_pool.float()).any()
    o = A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, 10)
    assert np.isfinite(o).all()


def test_large_scores_stay_finite():
    # scores spread over more than 800: exp without the max subtraction overflows
    shape, x = _inputs(21, Hq=2, Hkv=1, d=8, seed=11)
    q = (x.q.float() * 600).to(torch.bfloat16)
    o = A.decode_attention(q, x.k_pool, x.v_pool, x.table, 21)
    Kd, Vd = A.gather_cache(x.k_pool, x.v_pool, x.table, 21)
    s = Kd[0] @ q.double().numpy()[0] / math.sqrt(8)
    assert s.max() - s.min() > 800           # exp(800) overflows float64
    assert np.isfinite(o).all()
    # essentially all weight on the largest score
    np.testing.assert_allclose(o[0], Vd[0][int(np.argmax(s))], rtol=0,
                               atol=20 * math.exp(-(np.sort(s)[-1] - np.sort(s)[-2])) * 10 + 1e-12)
