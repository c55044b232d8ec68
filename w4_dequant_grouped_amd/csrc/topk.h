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

// ---------------------------------------------------------------------------
// top-k of one token's logits held by one wavefront
// ---------------------------------------------------------------------------
// vals[j] is the logit of expert e = lane + 64 j.  Chooses the k largest (ties
// to the lower expert) and writes them in ascending expert order to ids_out and
// w_out (and ids_lds when given), with the renormalised softmax weights
// exp(l - lmax) / (sum over the chosen).  No k sequential arg-max rounds: the
// k-th largest order key theta is found by bisection, each probe c costing one
// compare and one ballot count per register, f(c) = #{valid keys >= c}.  The
// bracket starts at [lo, hi]: hi is the largest key; lo is the smallest of the
// maxima of 8 disjoint lane groups (16 when k > 8), which are that many distinct
// entries, so f(lo) >= k.  The probes keep f(lo) >= k and theta <= hi, and stop
// early when f(c) == k: then no key lies in [c, theta), so the keys >= c are
// exactly the chosen ones.  For logits of a continuous distribution the bracket
// narrows to the gap between the k-th and (k+1)-th largest within a handful of
// probes (at most 32 in any case).  The entries above theta and the lowest-id
// entries equal to theta are chosen, and every chosen entry's rank in ascending
// expert order comes from the ballot masks, which are also returned in
// masks_out[j] (bit l: expert 64 j + l chosen) when given.  With w_out null the
// weights are neither computed nor written (ids only); ids_lds and w_lds receive
// second copies of the ids and weights when given.
template <int EPL>
__device__ __forceinline__ void wave_topk_select(const float (&vals)[EPL], int E, int k, int lane,
                                                 int32_t* __restrict__ ids_out,
                                                 float* __restrict__ w_out,
                                                 int32_t* ids_lds = nullptr,
                                                 float* w_lds = nullptr,
                                                 uint64_t* masks_out = nullptr) {
    uint32_t key[EPL];
    uint32_t g = 0u;                       // invalid entries hold key 0
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        key[j] = (lane + kWave * j < E) ? order_key(vals[j]) : 0u;
        g = key[j] > g ? key[j] : g;
    }
    // group maxima: 4 lanes (16 groups) or 8 lanes (8 groups); a group without a
    // valid entry has maximum 0, which makes lo = 0 and f(0) = E >= k
    auto gmax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    g = gmax(g, (uint32_t)dpp_i<kDppXor1>((int)g));
    g = gmax(g, (uint32_t)dpp_i<kDppXor2>((int)g));
    if (k <= 8) g = gmax(g, (uint32_t)dpp_i<kDppHalfMirror>((int)g));
    const uint32_t top = wave_max_u32(g);
    uint32_t lo = wave_min_u32(g), hi = top;
    while (lo < hi) {
        const uint32_t c = lo + ((hi - lo) >> 1) + 1u;   // lo < c <= hi
        int n = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] >= c));
        if (n < k) {
            hi = c - 1u;
        } else {
            lo = c;
            if (n == k) break;
        }
    }
    const uint32_t theta = lo;
    // chosen: key > theta, then key == theta in ascending expert order until k
    int above = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) above += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] > theta));
    const int need = k - above;
    bool sel[EPL];
    int eq_before = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const bool valid = lane + kWave * j < E;
        const bool eq = valid && key[j] == theta;
        const uint64_t m = __builtin_amdgcn_ballot_w64(eq);
        sel[j] = (valid && key[j] > theta) || (eq && eq_before + bits_below(m) < need);
        eq_before += __builtin_popcountll(m);
    }
    // weights: exp(l - lmax) over the chosen (an entry with the largest key is
    // always chosen)
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
        const uint64_t m = __builtin_amdgcn_ballot_w64(sel[j]);
        if (sel[j]) {
            const int rank = before + bits_below(m);
            ids_out[rank] = lane + kWave * j;
            if (ids_lds) ids_lds[rank] = lane + kWave * j;
            if (w_out) {
                w_out[rank] = p[j] * inv;
                if (w_lds) w_lds[rank] = p[j] * inv;
            }
        }
        if (masks_out && lane == 0) masks_out[j] = m;   // chosen experts 64 j .. 64 j + 63
        before += __builtin_popcountll(m);
    }
}

}  // namespace moe_w4
