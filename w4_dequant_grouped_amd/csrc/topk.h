// Top-k selection of one token's logits held by one wavefront.
#pragma once

#include "device.h"

namespace moe_w4 {

constexpr int kMaxTopK = 16;

// Order-preserving key of a float: larger float -> larger key; -0 counts as +0.
// The order is total (NaN sorts above +inf), so every lane agrees on the result
// and the chosen ids are always k distinct valid experts.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float order_key_inverse(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int bits_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Position of the r-th set bit (from 0) of a wavefront-uniform mask that has
// more than r set bits: the lanes with exactly r set bits below them run from
// just above the (r-1)-th set bit up to the r-th, so it is the highest of them.
__device__ __forceinline__ int nth_set_bit(uint64_t mask, int r) {
    return 63 - __builtin_clzll(__builtin_amdgcn_ballot_w64(bits_below(mask) == r));
}

// Order keys of one token's logits held by one wavefront: vals[j] is the logit
// of expert e = lane + 64 j; entries past E get key 0, below every valid key
// but the one of a negative NaN with every bit set.
template <int EPL>
__device__ __forceinline__ void wave_order_keys(const float (&vals)[EPL], int E, int lane,
                                                uint32_t (&key)[EPL]) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) key[j] = (lane + kWave * j < E) ? order_key(vals[j]) : 0u;
}

// ---------------------------------------------------------------------------
// the k largest keys of one token, held by one wavefront
// ---------------------------------------------------------------------------
// Chooses the k largest keys (ties to the lower expert) with no k sequential
// arg-max rounds: the k-th largest key theta is found by bisection, each probe c
// costing one compare and one ballot count per register, f(c) = #{keys >= c}.
// The bracket starts at [lo, hi]: hi is the largest key; lo is the smallest of
// the maxima of 8 disjoint lane groups (16 when k > 8), which are that many
// distinct entries, so f(lo) >= k.  The probes keep f(lo) >= k and theta <= hi,
// and stop early when f(c) == k: then no key lies in [c, theta), so the keys
// >= c are exactly the chosen ones and that probe's ballots are the answer.  For
// logits of a continuous distribution the bracket narrows to the gap between
// the k-th and (k+1)-th largest within a handful of probes, so this is the
// usual exit.  Otherwise (at most 32 probes) the bracket has closed on theta;
// then the keys above theta and the lowest-id keys equal to theta are chosen.
// sel[j] tells whether this lane's entry lane + 64 j is chosen and chosen[j] is
// its wavefront mask (bit l: expert 64 j + l).  Returns the largest key.
template <int EPL>
__device__ __forceinline__ uint32_t wave_topk_choose(const uint32_t (&key)[EPL], int E, int k, int lane,
                                                     bool (&sel)[EPL], uint64_t (&chosen)[EPL]) {
    uint32_t g = 0u;
#pragma unroll
    for (int j = 0; j < EPL; ++j) g = key[j] > g ? key[j] : g;
    // group maxima: 4 lanes (16 groups) or 8 lanes (8 groups); a group without a
    // valid entry has maximum 0, which makes lo = 0 and f(0) = E >= k
    auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    auto umin = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
    g = umax(g, (uint32_t)dpp_i<kDppXor1>((int)g));
    g = umax(g, (uint32_t)dpp_i<kDppXor2>((int)g));
    uint32_t gx = g, gn = g;     // extremes over the groups: g is uniform within a group
    if (k <= 8) {
        gx = umax(gx, (uint32_t)dpp_i<kDppHalfMirror>((int)gx));
        gn = gx;
    } else {
        gx = umax(gx, (uint32_t)dpp_i<kDppHalfMirror>((int)gx));
        gn = umin(gn, (uint32_t)dpp_i<kDppHalfMirror>((int)gn));
    }
    gx = umax(gx, (uint32_t)dpp_i<kDppMirror>((int)gx));
    gn = umin(gn, (uint32_t)dpp_i<kDppMirror>((int)gn));
    const uint32_t top = umax(umax((uint32_t)__builtin_amdgcn_readlane((int)gx, 0), (uint32_t)__builtin_amdgcn_readlane((int)gx, 16)),
                              umax((uint32_t)__builtin_amdgcn_readlane((int)gx, 32), (uint32_t)__builtin_amdgcn_readlane((int)gx, 48)));
    uint32_t lo = umin(umin((uint32_t)__builtin_amdgcn_readlane((int)gn, 0), (uint32_t)__builtin_amdgcn_readlane((int)gn, 16)),
                       umin((uint32_t)__builtin_amdgcn_readlane((int)gn, 32), (uint32_t)__builtin_amdgcn_readlane((int)gn, 48)));
    uint32_t hi = top;
    bool exact = false;
    while (lo < hi) {
        const uint32_t c = lo + ((hi - lo) >> 1) + 1u;   // lo < c <= hi
        int n = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] >= c));
        if (n < k) {
            hi = c - 1u;
        } else {
            lo = c;
            if (n == k) {
                exact = true;
                break;
            }
        }
    }
    const uint32_t theta = lo;
    if (exact) {
        // f(theta) == k; theta >= 1, so no entry past E is counted
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            sel[j] = key[j] >= theta;
            chosen[j] = __builtin_amdgcn_ballot_w64(sel[j]);
        }
    } else {
        int need = k;
        bool eq[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const bool valid = lane + kWave * j < E;
            sel[j] = valid && key[j] > theta;
            eq[j] = valid && key[j] == theta;
            need -= __builtin_popcountll(__builtin_amdgcn_ballot_w64(sel[j]));
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(eq[j]);
            sel[j] = sel[j] || (eq[j] && bits_below(m) < need);
            need -= __builtin_popcountll(m);
            chosen[j] = __builtin_amdgcn_ballot_w64(sel[j]);
        }
    }
    return top;
}

// ---------------------------------------------------------------------------
// top-k of one token's logits held by one wavefront
// ---------------------------------------------------------------------------
// vals[j] is the logit of expert e = lane + 64 j.  Chooses the k largest (ties
// to the lower expert, see wave_topk_choose) and writes them in ascending expert
// order to ids_out and w_out (and ids_lds when given), with the renormalised
// softmax weights exp(l - lmax) / (sum over the chosen); an entry with the
// largest key is always chosen, so lmax is the bracket's top.  Every chosen
// entry's rank in ascending expert order comes from the ballot masks, which are
// also returned in masks_out[j] (bit l: expert 64 j + l chosen) when given.  With
// w_out null the weights are neither computed nor written (ids only), and with
// ids_out null the ids are not written either; ids_lds and w_lds receive second
// copies of the ids and weights when given.
template <int EPL>
__device__ __forceinline__ void wave_topk_select(const float (&vals)[EPL], int E, int k, int lane,
                                                 int32_t* __restrict__ ids_out,
                                                 float* __restrict__ w_out,
                                                 int32_t* ids_lds = nullptr,
                                                 float* w_lds = nullptr,
                                                 uint64_t* masks_out = nullptr,
                                                 uint8_t* __restrict__ ids8_out = nullptr) {
    uint32_t key[EPL];
    wave_order_keys<EPL>(vals, E, lane, key);
    bool sel[EPL];
    uint64_t chosen[EPL];
    const uint32_t top = wave_topk_choose<EPL>(key, E, k, lane, sel, chosen);
    float p[EPL];
    float inv = 0.f;
    if (w_out) {
        const float vmax = order_key_inverse(top);
        float local = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            p[j] = sel[j] ? expf(vals[j] - vmax) : 0.f;
            local += p[j];
        }
        inv = 1.0f / wave_sum(local);
    }
    int before = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        if (sel[j]) {
            const int rank = before + bits_below(chosen[j]);
            if (ids_out) ids_out[rank] = lane + kWave * j;
            if (ids_lds) ids_lds[rank] = lane + kWave * j;
            if (ids8_out) ids8_out[rank] = (uint8_t)(lane + kWave * j);   // E <= 256
            if (w_out) {
                w_out[rank] = p[j] * inv;
                if (w_lds) w_lds[rank] = p[j] * inv;
            }
        }
        if (masks_out && lane == 0) masks_out[j] = chosen[j];   // chosen experts 64 j .. 64 j + 63
        before += __builtin_popcountll(chosen[j]);
    }
}

// The expert of the r-th chosen entry in ascending expert order (r < k): the
// same choice as wave_topk_select, for a caller that needs one id, with no
// writes and no LDS.
template <int EPL>
__device__ __forceinline__ int wave_topk_nth(const float (&vals)[EPL], int E, int k, int lane, int r) {
    uint32_t key[EPL];
    wave_order_keys<EPL>(vals, E, lane, key);
    bool sel[EPL];
    uint64_t chosen[EPL];
    wave_topk_choose<EPL>(key, E, k, lane, sel, chosen);
    // the mask that holds the r-th chosen entry, and r's rank within it
    uint64_t m = chosen[0];
    int base = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int cnt = __builtin_popcountll(chosen[j]);
        if (!found) {
            if (r < cnt) {
                m = chosen[j];
                base = kWave * j;
                found = true;
            } else {
                r -= cnt;
            }
        }
    }
    return base + nth_set_bit(m, r);
}

}  // namespace moe_w4
