"""Pins for the Gated DeltaNet oracle: each checks it against something other than
itself.

beta = 0 leaves only the decay (a closed form); alpha = beta = 1 with orthonormal
keys stores every (key, value) pair exactly (exact recall); a repeated key is
overwritten; the paper's product form S (alpha (I - beta k k^T)) + beta v k^T with
explicit matrices; linearity in (initial state, values); a sequence split in two
with the state carried over; the value-head to key-head mapping.  A slip (a
missing alpha on the correction, the update before the read, a transposed state,
q and k swapped, the wrong head mapping) fails one of them.
"""
import numpy as np
import pytest
import torch

from oracle import gdn_oracle as D
from w4_dequant_grouped_amd import synth_gdn as SG


def _draw(T=9, Hv=4, Hk=2, d=8, seed=0):
    return SG.draw_gdn(SG.GdnShape(T=T, n_v_heads=Hv, n_k_heads=Hk, dim=d), seed)


def test_beta_zero_is_pure_decay():
    x = _draw(seed=1)
    beta = torch.zeros_like(x.beta)
    o, S = D.gdn_scan(x.q, x.k, x.v, x.g, beta, x.state)
    S0 = x.state.double().numpy()
    cum = np.cumsum(x.g.double().numpy(), axis=0)            # [T][Hv]
    Q = x.q.double().numpy()
    for t in range(x.q.shape[0]):
        for h in range(4):
            ref = np.exp(cum[t, h]) * S0[h] @ Q[t, h // 2]
            np.testing.assert_allclose(o[t, h], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, np.exp(cum[-1])[:, None, None] * S0, rtol=0, atol=1e-12)


def test_exact_recall_of_orthonormal_keys():
    d, T = 8, 5
    rng = np.random.default_rng(2)
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = torch.tensor(basis[:T][:, None, :], dtype=torch.float64)        # [T][1][d], orthonormal
    v = torch.tensor(rng.standard_normal((T, 1, d)))
    q = torch.tensor(rng.standard_normal((T, 1, d)))
    g = torch.zeros((T, 1), dtype=torch.float64)                        # alpha = 1
    beta = torch.ones((T, 1), dtype=torch.float64)
    S0 = torch.zeros((1, d, d), dtype=torch.float64)
    o, S = D.gdn_scan(q, k, v, g, beta, S0)
    # S_T = sum_i v_i k_i^T: every stored key reads back its value
    for i in range(T):
        np.testing.assert_allclose(S[0] @ basis[i], v[i, 0].numpy(), rtol=0, atol=1e-12)
    # o_t = sum_{i <= t} v_i (k_i . q_t)
    for t in range(T):
        ref = sum(v[i, 0].numpy() * (basis[i] @ q[t, 0].numpy()) for i in range(t + 1))
        np.testing.assert_allclose(o[t, 0], ref, rtol=0, atol=1e-12)


def test_repeated_key_is_overwritten():
    d = 8
    rng = np.random.default_rng(3)
    kk = rng.standard_normal(d)
    kk /= np.linalg.norm(kk)
    k = torch.tensor(np.stack([kk, kk])[:, None, :])
    v = torch.tensor(rng.standard_normal((2, 1, d)))
    q = torch.tensor(np.stack([kk, kk])[:, None, :])
    g = torch.zeros((2, 1), dtype=torch.float64)
    beta = torch.ones((2, 1), dtype=torch.float64)
    S0 = torch.tensor(rng.standard_normal((1, d, d)))
    o, S = D.gdn_scan(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o[0, 0], v[0, 0].numpy(), rtol=0, atol=1e-12)   # S_1 k = v_1
    np.testing.assert_allclose(o[1, 0], v[1, 0].numpy(), rtol=0, atol=1e-12)   # replaced by v_2


def test_matches_the_product_form_with_explicit_matrices():
    x = _draw(T=7, Hv=2, Hk=1, d=6, seed=4)
    o, S = D.gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.state)
    Q, K, V = (t.double().numpy() for t in (x.q, x.k, x.v))
    G, B = x.g.double().numpy(), x.beta.double().numpy()
    I = np.eye(6)
    for h in range(2):
        Sh = x.state[h].double().numpy()
        for t in range(7):
            kt = K[t, 0][:, None]
            a = np.exp(G[t, h])
            Sh = Sh @ (a * (I - B[t, h] * kt @ kt.T)) + B[t, h] * V[t, h][:, None] @ kt.T
            np.testing.assert_allclose(o[t, h], Sh @ Q[t, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(S[h], Sh, rtol=0, atol=1e-12)


def test_linear_in_initial_state_and_values():
    x = _draw(seed=5)
    o1, S1 = D.gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.state)
    o2, S2 = D.gdn_scan(x.q, x.k, 3 * x.v.double(), x.g, x.beta, 3 * x.state.double())
    np.testing.assert_allclose(o2, 3 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, 3 * S1, rtol=1e-12, atol=1e-12)


def test_split_sequence_with_state_carried_over():
    x = _draw(T=11, seed=6)
    o, S = D.gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.state)
    oa, Sa = D.gdn_scan(x.q[:4], x.k[:4], x.v[:4], x.g[:4], x.beta[:4], x.state)
    ob, Sb = D.gdn_scan(x.q[4:], x.k[4:], x.v[4:], x.g[4:], x.beta[4:], torch.tensor(Sa))
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Sb, S, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hv,Hk", [(4, 2), (6, 3), (4, 1)])
def test_head_mapping_matches_repeated_heads(Hv, Hk):
    x = _draw(Hv=Hv, Hk=Hk, seed=7)
    rep = Hv // Hk
    o1, S1 = D.gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.state)
    o2, S2 = D.gdn_scan(x.q.repeat_interleave(rep, dim=1), x.k.repeat_interleave(rep, dim=1),
                        x.v, x.g, x.beta, x.state)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_q_and_k_play_different_roles():
    # swapping q and k changes the result (the read uses q, the write uses k)
    x = _draw(seed=8)
    o1, _ = D.gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.state)
    o2, _ = D.gdn_scan(x.k, x.q, x.v, x.g, x.beta, x.state)
    assert np.abs(o1 - o2).max() > 1e-3
