// Device-side helpers shared by the gfx950 kernels of the W4 MoE block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe_w4 {

constexpr int kWave = 64;
constexpr int kGroup = 64;   // quantisation group along K

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// --- scalar conversions ----------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// Two floats -> one dword of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// silu(z) = z / (1 + e^-z) from the hardware exp2 and reciprocal (v_exp_f32,
// v_rcp_f32: about one ulp each, five VALU ops in all instead of an IEEE
// division).  Every caller rounds the result to bf16, far coarser than that.
// Limits: e^-z overflows to +inf for very negative z, giving z * 0 = -0; for
// large z it underflows to 0, giving z.
__device__ __forceinline__ float silu(float z) {
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * z);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// --- 4-bit code unpacking -----------------------------------------------------
// A dword of packed codes holds k = 0..7 of a row: byte i = (c[2i+1] << 4) | c[2i].

// Dequantise 8 codes to bf16 with w = c * s + b (fp32 FMA, one RNE rounding).
// Natural k order: element i of the result is k = i.
__device__ __forceinline__ bf16x8 dequant8(uint32_t d, float s, float b) {
    const uint32_t lo = d & 0x0F0F0F0Fu;          // c0 c2 c4 c6 in bytes 0..3
    const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;   // c1 c3 c5 c7
    float w0 = fmaf((float)(lo & 0xFF), s, b);
    float w1 = fmaf((float)(hi & 0xFF), s, b);
    float w2 = fmaf((float)((lo >> 8) & 0xFF), s, b);
    float w3 = fmaf((float)((hi >> 8) & 0xFF), s, b);
    float w4 = fmaf((float)((lo >> 16) & 0xFF), s, b);
    float w5 = fmaf((float)((hi >> 16) & 0xFF), s, b);
    float w6 = fmaf((float)(lo >> 24), s, b);
    float w7 = fmaf((float)(hi >> 24), s, b);
    u32x4 p = {pack_bf16x2(w0, w1), pack_bf16x2(w2, w3), pack_bf16x2(w4, w5), pack_bf16x2(w6, w7)};
    return __builtin_bit_cast(bf16x8, p);
}

// (a & m) | c in one instruction.  gfx9 VOP3 may read one SGPR, so the constant
// c is kept in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Per (row, group) constants of the fp16-magic dequantisation below.
struct DqConst {
    float s0, b0;   // nibble in bits 0..3 of a half: value 1024 + c
    float s1, b1;   // nibble in bits 4..7 of a half: value 1024 + 16 c
};
__device__ __forceinline__ DqConst make_dq(float s, float b) {
    // b - 1024 s and b - 64 s are exact in fp32 for bf16 s and b of similar
    // magnitude, so each weight below is c*s + b rounded once
    return DqConst{s, fmaf(-1024.0f, s, b), s * 0.0625f, fmaf(-64.0f, s, b)};
}

// Dequantise 8 codes (one dword, natural k order) to bf16 w = c*s + b.
// fp16(1024 + c) has bit pattern 0x6400 | c and fp16(1024 + 16c) is 0x6400 | (c << 4),
// so one AND-OR per pair of codes builds exact fp16 operands and v_fma_mix_f32
// applies the affine map in fp32 with a single rounding: 17 VALU ops per 8 weights.
__device__ __forceinline__ bf16x8 dequant8_mix(uint32_t d, const DqConst& q, uint32_t magic) {
    const uint32_t t = d >> 8;
    const f16x2 h0 = __builtin_bit_cast(f16x2, and_or(d, 0x000F000Fu, magic));   // c0, c4
    const f16x2 h1 = __builtin_bit_cast(f16x2, and_or(d, 0x00F000F0u, magic));   // c1, c5 (x16)
    const f16x2 h2 = __builtin_bit_cast(f16x2, and_or(t, 0x000F000Fu, magic));   // c2, c6
    const f16x2 h3 = __builtin_bit_cast(f16x2, and_or(t, 0x00F000F0u, magic));   // c3, c7 (x16)
    const float w0 = fmaf((float)h0.x, q.s0, q.b0), w4 = fmaf((float)h0.y, q.s0, q.b0);
    const float w1 = fmaf((float)h1.x, q.s1, q.b1), w5 = fmaf((float)h1.y, q.s1, q.b1);
    const float w2 = fmaf((float)h2.x, q.s0, q.b0), w6 = fmaf((float)h2.y, q.s0, q.b0);
    const float w3 = fmaf((float)h3.x, q.s1, q.b1), w7 = fmaf((float)h3.y, q.s1, q.b1);
    u32x4 p = {pack_bf16x2(w0, w1), pack_bf16x2(w2, w3), pack_bf16x2(w4, w5), pack_bf16x2(w6, w7)};
    return __builtin_bit_cast(bf16x8, p);
}

// Codes as bf16 "magic" pairs: bf16(128 + c) has bit pattern 0x4300 | c, exactly.
// Pair j (j = 0..3) of a dword holds (c[j], c[j+4]) in (bits 0..15, bits 16..31).
// `magic` is 0x43004300 held in a register (one AND-OR per pair).
__device__ __forceinline__ uint32_t magic_pair(uint32_t d, int j, uint32_t magic) {
    return and_or(d >> (4 * j), 0x000F000Fu, magic);
}

// Reorder 8 consecutive bf16 values x0..x7 (given as 4 dwords of natural pairs)
// into the pairs (x[j], x[j+4]) that line up with magic_pair(d, j).
__device__ __forceinline__ uint32_t interleave_pair(uint32_t a, uint32_t b, int hi) {
    // hi = 0: (lo16(a), lo16(b)); hi = 1: (hi16(a), hi16(b))
    return hi ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
}

// fp32 dot of two bf16 pairs plus accumulator.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// --- wave reductions ----------------------------------------------------------
// Within each row of 16 lanes, DPP moves (quad_perm xor 1, xor 2, row_half_mirror,
// row_mirror) pair every lane with partners covering the whole row; four
// readlanes then combine the rows.  No LDS traffic, fixed summation order.
// Every control used here reads a lane of the same row, so the bound-control bit
// never takes effect with all lanes active; it is set because it lets the
// compiler fold each move into the add that consumes it (v_add_f32_dpp).

template <int ctrl>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, true);
}
template <int ctrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<ctrl>(__float_as_int(v)));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i within 16

// Every lane receives the sum of its row of 16 lanes.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return v;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over the wavefront, returned (uniform) in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Maximum and minimum of an unsigned 32-bit value over the wavefront, returned
// (uniform) in every lane.
template <bool kMax>
__device__ __forceinline__ uint32_t wave_extreme_u32(uint32_t v) {
    auto pick = [](uint32_t a, uint32_t b) { return kMax ? (a > b ? a : b) : (a < b ? a : b); };
    v = pick(v, (uint32_t)dpp_i<kDppXor1>((int)v));
    v = pick(v, (uint32_t)dpp_i<kDppXor2>((int)v));
    v = pick(v, (uint32_t)dpp_i<kDppHalfMirror>((int)v));
    v = pick(v, (uint32_t)dpp_i<kDppMirror>((int)v));
    const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
    return pick(pick(r0, r1), pick(r2, r3));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_extreme_u32<true>(v); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_extreme_u32<false>(v); }

// --- memory -------------------------------------------------------------------

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace moe_w4
