// Wavefront-per-row W4 dot products of the decode kernels.
//
// A lane holds 32 consecutive codes (one 128-bit load) and dots them against
// activation rows with the per-group affine form
//   sum_k (c s + b) x_k = s * sum_k (128 + c) x_k + (b - 128 s) * sum_k x_k,
// where bf16(128 + c) has the bit pattern 0x4300 | c, so the codes become bf16
// operands of v_dot2_f32_bf16 after one AND-OR per pair.
#pragma once

#include "device.h"

namespace moe_w4 {

// 32 bf16 of a row (64 bytes at p) -> 16 dwords paired as (x[j], x[j+4]) per 8,
// plus their sum.
__device__ __forceinline__ void interleave32(const u32x4 (&v)[4], uint32_t (&xi)[16], float& sum) {
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        xi[4 * b + 0] = interleave_pair(v[b].x, v[b].z, 0);
        xi[4 * b + 1] = interleave_pair(v[b].x, v[b].z, 1);
        xi[4 * b + 2] = interleave_pair(v[b].y, v[b].w, 0);
        xi[4 * b + 3] = interleave_pair(v[b].y, v[b].w, 1);
        s = dot2_bf16(v[b].x, 0x3F803F80u, s);
        s = dot2_bf16(v[b].y, 0x3F803F80u, s);
        s = dot2_bf16(v[b].z, 0x3F803F80u, s);
        s = dot2_bf16(v[b].w, 0x3F803F80u, s);
    }
    sum = s;
}

__device__ __forceinline__ void load64(const uint16_t* p, u32x4 (&v)[4]) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = q[b];
}

// sum_k (128 + c_k) x_k over 32 codes (4 dwords) and the matching interleaved x.
__device__ __forceinline__ float dot32_magic(const u32x4& c, const uint32_t (&xi)[16]) {
    const uint32_t magic = 0x43004300u;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a0 = dot2_bf16(magic_pair(c.x, j, magic), xi[j], a0);
        a1 = dot2_bf16(magic_pair(c.y, j, magic), xi[4 + j], a1);
        a0 = dot2_bf16(magic_pair(c.z, j, magic), xi[8 + j], a0);
        a1 = dot2_bf16(magic_pair(c.w, j, magic), xi[12 + j], a1);
    }
    return a0 + a1;
}

}  // namespace moe_w4
