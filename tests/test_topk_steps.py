"""The wavefront top-k of csrc/topk.h, step by step on the CPU, against brute force.

This checks the selection algorithm's design, not the HIP code (the GPU parity
tests compare the kernels with the oracle).  The steps modelled here, in the
kernel's order and notation:

- order keys: -0 counts as +0, NaN sorts above +inf, entries past E get key 0;
- the bracket: lo = the smallest of the maxima of 8 lane groups of 8 lanes (16
  groups of 4 when k > 8), hi = the largest key, so f(lo) >= k;
- bisection on f(c) = #{keys >= c}, probe c = lo + (hi - lo) // 2 + 1, stopping
  when f(c) == k (then the keys >= c are the chosen set);
- otherwise the tie path at theta = lo: keys above theta, then keys equal to
  theta in ascending expert order up to k;
- the expert of slot r (the r-th chosen in ascending id order) as the highest
  lane with exactly r chosen bits below it in the mask that holds it.

Expert e sits in lane e % 64 of register e // 64, as in the kernels.
"""
import struct

import numpy as np
import pytest


def order_key(v: float) -> int:
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    if b == 0x80000000:
        b = 0
    return (~b) & 0xFFFFFFFF if b & 0x80000000 else b | 0x80000000


def wave_topk(vals, E: int, k: int):
    """Chosen experts (ascending), the largest key, slot experts and the probe count."""
    epl = max(1, (E + 63) // 64)
    key = np.zeros((epl, 64), dtype=np.int64)
    valid = np.zeros((epl, 64), dtype=bool)
    for e in range(E):
        key[e // 64, e % 64] = order_key(float(np.float32(vals[e])))
        valid[e // 64, e % 64] = True
    lane_max = key.max(axis=0)
    group = 4 if k > 8 else 8
    gmax = lane_max.reshape(64 // group, group).max(axis=1)
    lo, hi = int(gmax.min()), int(gmax.max())
    top = hi
    exact, probes = False, 0
    while lo < hi:
        c = lo + ((hi - lo) >> 1) + 1
        n = int((key >= c).sum())
        probes += 1
        if n < k:
            hi = c - 1
        else:
            lo = c
            if n == k:
                exact = True
                break
    theta = lo
    if exact:
        sel = key >= theta
        assert not (sel & ~valid).any(), "an entry past E was chosen"
    else:
        need = k
        sel = valid & (key > theta)
        eq = valid & (key == theta)
        need -= int(sel.sum())
        for j in range(epl):
            below = np.concatenate([[0], np.cumsum(eq[j])[:-1]])
            sel[j] = sel[j] | (eq[j] & (below < need))
            need -= int(eq[j].sum())
    masks = [sum(1 << l for l in range(64) if sel[j, l]) for j in range(epl)]
    slots = []
    for r in range(k):
        rr, m, base = r, masks[0], 0
        for j in range(epl):
            cnt = bin(masks[j]).count("1")
            if rr < cnt:
                m, base = masks[j], 64 * j
                break
            rr -= cnt
        lanes = [l for l in range(64) if bin(m & ((1 << l) - 1)).count("1") == rr]
        slots.append(base + max(lanes))
    chosen = sorted(l + 64 * j for j in range(epl) for l in range(64) if sel[j, l])
    return chosen, top, slots, probes


def brute_force(vals, E: int, k: int):
    keys = [order_key(float(np.float32(v))) for v in vals[:E]]
    order = sorted(range(E), key=lambda e: (-keys[e], e))
    return sorted(order[:k]), max(keys)


def draw(kind: int, E: int, rng):
    if kind == 0:
        return rng.standard_normal(E).astype(np.float32)
    if kind == 1:                                    # many ties
        return rng.integers(-3, 4, E).astype(np.float32)
    if kind == 2:                                    # all equal
        return np.full(E, 1.5, np.float32)
    if kind == 3:                                    # NaN, -0, +0, -inf
        v = rng.standard_normal(E).astype(np.float32)
        v[rng.integers(0, E, 3)] = np.nan
        v[rng.integers(0, E, 2)] = -0.0
        v[rng.integers(0, E, 2)] = 0.0
        v[rng.integers(0, E, 2)] = -np.inf
        return v
    if kind == 4:                                    # arbitrary bit patterns
        bits = rng.integers(0, 2 ** 32, E, dtype=np.uint64).astype(np.uint32)
        return np.frombuffer(bits.tobytes(), np.float32).copy()
    return (rng.standard_normal(E) * 3 + 1).astype(np.float32)


@pytest.mark.parametrize("kind", range(6))
def test_steps_match_brute_force(kind):
    rng = np.random.default_rng(100 + kind)
    for _ in range(500):
        E = int(rng.choice([1, 2, 5, 16, 63, 64, 65, 100, 128, 200, 256]))
        k = int(rng.integers(1, min(16, E) + 1))
        v = draw(kind, E, rng)
        chosen, top, slots, probes = wave_topk(v, E, k)
        ref, ref_top = brute_force(v, E, k)
        assert chosen == ref, (kind, E, k)
        assert top == ref_top
        assert slots == ref, "slot r must hold the r-th chosen expert in ascending id"
        assert probes <= 32


def test_probe_count_on_router_logits():
    # 256 normal logits, top-8: the bracket and the early exit keep the search short
    rng = np.random.default_rng(7)
    probes = [wave_topk(rng.standard_normal(256).astype(np.float32) * 2.26, 256, 8)[3]
              for _ in range(500)]
    assert np.mean(probes) < 6.0


def test_exact_exit_on_a_probe_equal_to_the_kth_key():
    # E=16, k=2: the lane groups of 8 beyond lane 15 hold no entry, so lo = 0 and the
    # first probe is c = hi // 2 + 1.  Expert 3 gets exactly that key (the float whose
    # order key is c) and expert 9 the largest, so the search stops at once on a probe
    # that equals the k-th key: the chosen set must include it (keys >= c).
    hi = order_key(1.0)
    c = hi // 2 + 1
    bits = (~c) & 0xFFFFFFFF                 # keys below 2^31 are negative floats: key = ~bits
    v = np.full(16, -1e30, np.float32)
    v[9] = 1.0
    v[3] = np.frombuffer(np.uint32(bits).tobytes(), np.float32)[0]
    assert order_key(float(v[3])) == c
    chosen, _, slots, probes = wave_topk(v, 16, 2)
    assert probes == 1
    assert chosen == brute_force(v, 16, 2)[0] == [3, 9]
    assert slots == [3, 9]
