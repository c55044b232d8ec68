// Top-k selection of one token's logits held by one wavefront.
#pragma once

#include "device.h"

namespace moe_w4 {

constexpr int kMaxTopK = 16;

// ---------------------------------------------------------------------------
// top-k of one token's logits held by one wavefront
// ---------------------------------------------------------------------------
// vals[j] is the logit of expert e = lane + 64 * j (or -inf past E).  Chooses the
// k largest (ties -> lower expert index); lane r < k writes chosen entry r, at its
// rank in ascending expert order, to ids_out / w_out (global) and to ids_lds when
// given; the weights are the renormalised softmax exp(l - lmax) / sum over the
// chosen.  Returns, in every lane, the id chosen in round `lane` (-1 if lane >= k).
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

template <int EPL>
__device__ __forceinline__ int wave_topk(float (&vals)[EPL], int E, int k, int lane,
                         int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                         int32_t* ids_lds) {
    int sel_e[kMaxTopK];
    float sel_v[kMaxTopK];
    // 64-bit key: order key of the logit, then ~expert so that equal logits
    // prefer the lower expert; 0 marks an absent or already chosen entry
    uint64_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + kWave * j;
        key[j] = (e < E) ? (((uint64_t)order_key(vals[j]) << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
    }
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (r >= k) { sel_e[r] = 0x7FFFFFFF; sel_v[r] = 0.f; continue; }
        uint64_t best = 0ull;
#pragma unroll
        for (int j = 0; j < EPL; ++j) best = key[j] > best ? key[j] : best;
        best = wave_max_u64(best);
        const int be = (int)(~(uint32_t)best);
        sel_e[r] = be;
        sel_v[r] = order_key_inverse((uint32_t)(best >> 32));
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + kWave * j == be) key[j] = 0ull;
    }
    // renormalised softmax over the chosen logits (the full-softmax denominator cancels)
    const float vmax = sel_v[0];
    float p[kMaxTopK];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        p[r] = (r < k) ? expf(sel_v[r] - vmax) : 0.f;
        psum += p[r];
    }
    const float inv = 1.0f / psum;
    int mine = -1;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (r >= k) break;
        int rank = 0;
#pragma unroll
        for (int q = 0; q < kMaxTopK; ++q) rank += (q < k && sel_e[q] < sel_e[r]) ? 1 : 0;
        if (lane == r) {
            mine = sel_e[r];
            ids_out[rank] = sel_e[r];
            w_out[rank] = p[r] * inv;
            if (ids_lds) ids_lds[rank] = sel_e[r];
        }
    }
    return mine;
}

}  // namespace moe_w4
