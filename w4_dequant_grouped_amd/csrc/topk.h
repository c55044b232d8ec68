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
// exp(l - lmax) / (sum over the chosen).  No k sequential arg-max rounds: a
// bitwise binary search on the order keys finds the k-th largest key theta (32
// steps of one compare and one ballot count each); the entries above theta and
// the lowest-id entries equal to theta are chosen, and every chosen entry's rank
// in ascending expert order comes from the ballot masks, which are also
// returned in masks_out[j] (bit l: expert 64 j + l chosen) when given.
template <int EPL>
__device__ __forceinline__ void wave_topk_select(const float (&vals)[EPL], int E, int k, int lane,
                                                 int32_t* __restrict__ ids_out,
                                                 float* __restrict__ w_out,
                                                 int32_t* ids_lds = nullptr,
                                                 uint64_t* masks_out = nullptr) {
    uint32_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) key[j] = (lane + kWave * j < E) ? order_key(vals[j]) : 0u;
    // theta: the largest value with #{key >= theta} >= k
    uint32_t theta = 0u;
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = theta | (1u << b);
        int n = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] >= c));
        if (n >= k) theta = c;
    }
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
    // weights: exp(l - lmax) over the chosen (the largest logit is always chosen)
    uint32_t kmax = 0u;
#pragma unroll
    for (int j = 0; j < EPL; ++j) kmax = (sel[j] && key[j] > kmax) ? key[j] : kmax;
    kmax = (uint32_t)(wave_max_u64((uint64_t)kmax));
    const float vmax = order_key_inverse(kmax);
    float p[EPL];
    float local = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        p[j] = sel[j] ? expf(vals[j] - vmax) : 0.f;
        local += p[j];
    }
    const float inv = 1.0f / wave_sum(local);
    int before = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(sel[j]);
        if (sel[j]) {
            const int rank = before + bits_below(m);
            ids_out[rank] = lane + kWave * j;
            w_out[rank] = p[j] * inv;
            if (ids_lds) ids_lds[rank] = lane + kWave * j;
        }
        if (masks_out && lane == 0) masks_out[j] = m;   // chosen experts 64 j .. 64 j + 63
        before += __builtin_popcountll(m);
    }
}

}  // namespace moe_w4
