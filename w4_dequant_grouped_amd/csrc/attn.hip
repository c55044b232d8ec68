// Decode attention over a paged KV cache (one query token), gfx950.
//
// The model's full-attention layers have 16 query heads over two key/value heads
// ("Perplexity's Lily brings fast local AI to Apple silicon Macs", section "A 35B
// Model Built for Local Memory").  Decode at long context is a stream over the
// cached keys and values, and the pages name the two changes that pay there: the
// query heads of a group are packed so that each cached row is read once, and the
// cache is laid out in fixed-size blocks ("Perplexity built an inference engine
// for one model, one chip", paragraph 3; "Perplexity's Lily ...", section "Where
// the Engine Gains Speed").
//
// Layout: k_pool / v_pool bf16 [P][Hkv][64][128]; logical block i of the context
// is physical block table[i]; one 64 x 128 block of one head is 16 KB contiguous.
//
//   k_attn_split   grid (splits, Hkv), four wavefronts.  A workgroup owns a run of
//                  blocks of one key/value head; each wavefront takes one block at a
//                  time.  s = K q for the G query heads of the group is one
//                  16x16x32 bf16 MFMA chain per 16 keys (keys are the M side, query
//                  heads the N side, so a K row is read once for all G heads); the
//                  online softmax runs on the MFMA output layout; p V runs on the
//                  VALU with each lane owning 8 columns of d for 16 of the keys,
//                  two keys per v_dot2_f32_bf16 (V rows are d-contiguous, the
//                  wrong way round for an MFMA operand).  The four wavefronts'
//                  states are merged in LDS and written as one partial (max,
//                  sum, numerator) per head.
//   k_attn_combine grid (Hq, 8): merges the partials of every split.
#include "device.h"
#include "kernels.h"

namespace moe_w4 {

constexpr int kAttnD = 128;
constexpr int kAttnB = 64;
constexpr int kAttnWaves = 4;
constexpr int kAttnHeads = 16;       // N side of the MFMA: query heads per group, padded

template <int GM>
struct AttnLds {
    float p[kAttnWaves][kAttnB][kAttnHeads];   // softmax numerators, [key][head], per wavefront
    float corr[kAttnWaves][kAttnHeads];        // rescale of the running state, per head
    float m[kAttnWaves][kAttnHeads];
    float l[kAttnWaves][kAttnHeads];
    float acc[kAttnWaves][GM][kAttnD];
};

// GM: query heads per group the accumulators are sized for (a.G <= GM).
template <int GM>
__global__ __launch_bounds__(256, GM <= 8 ? 2 : 1) void k_attn_split(AttnArgs a) {
    __shared__ AttnLds<GM> sm;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15, r4 = lane >> 4;
    const int kvh = blockIdx.y;
    const int G = a.G;
    const int nblk = (a.n_ctx + kAttnB - 1) / kAttnB;
    const int b0 = blockIdx.x * a.bpw;
    const int b1 = min(b0 + a.bpw, nblk);

    // B operand: query head kvh*G + r16 (zero past G), d = 32 ks + 8 r4 .. +8
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r16 < G)
            v = load_u32x4(a.q + (size_t)(kvh * G + r16) * kAttnD + 32 * ks + 8 * r4);
        qf[ks] = __builtin_bit_cast(bf16x8, v);
    }

    float m_run = -INFINITY;   // running max of head r16's raw scores (same in its 4 lanes)
    float l_run = 0.f;         // this lane's share of head r16's running sum
    float acc[GM][8];          // p V: heads 0..GM-1, d = 8 r16 + e, keys with phase r4
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

    for (int b = b0 + wave; b < b1; b += kAttnWaves) {
        const int phys = min(max(a.table[b], 0), a.n_pool - 1);
        const size_t base = ((size_t)phys * a.Hkv + kvh) * kAttnB * kAttnD;
        const uint16_t* kb = a.k_pool + base;
        const uint16_t* vb = a.v_pool + base;
        const int nvalid = min(kAttnB, a.n_ctx - b * kAttnB);
        // A operand: key 16 mt + r16, d = 32 ks + 8 r4 .. +8
        bf16x8 kf[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kf[mt][ks] = __builtin_bit_cast(
                    bf16x8, load_u32x4(kb + (size_t)(16 * mt + r16) * kAttnD + 32 * ks + 8 * r4));
        // V: key 4 j + r4, d = 8 r16 .. +8 (four rows of 256 B per instruction)
        u32x4 vf[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) vf[j] = load_u32x4(vb + (size_t)(4 * j + r4) * kAttnD + 8 * r16);

        // raw scores: lane holds keys 16 mt + 4 r4 + i of head r16
        f32x4 sc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                sc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt][ks], qf[ks], sc[mt], 0, 0, 0);
        }
        // slots past the context are masked by position (whatever they hold)
        float smax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = 16 * mt + 4 * r4 + i;
                const float v = key < nvalid ? sc[mt][i] : -INFINITY;
                sc[mt][i] = v;
                smax = fmaxf(smax, v);
            }
        smax = fmaxf(smax, __shfl_xor(smax, 16, kWave));
        smax = fmaxf(smax, __shfl_xor(smax, 32, kWave));
        const float m_new = fmaxf(m_run, smax);          // finite: the block has a valid key
        const float corr = exp2f((m_run - m_new) * a.c);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = exp2f((sc[mt][i] - m_new) * a.c);
                lsum += p;
                sm.p[wave][16 * mt + 4 * r4 + i][r16] = p;
            }
        l_run = l_run * corr + lsum;
        if (r4 == 0) sm.corr[wave][r16] = corr;

        // p V (the LDS writes above come from this wavefront, in order)
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            const float cg = sm.corr[wave][g];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] *= cg;
        }
        // keys 4j + r4 and 4j + 4 + r4 in pairs: one v_dot2_f32_bf16 per head and
        // column takes both (p rounded to bf16, V pairs gathered by byte permutes)
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            const int ka = 4 * j + r4, kb = ka + 4;
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 va = ka < nvalid ? vf[j] : z;
            const u32x4 vb = kb < nvalid ? vf[j + 1] : z;
            const uint32_t vp[8] = {
                __builtin_amdgcn_perm(vb.x, va.x, 0x05040100u), __builtin_amdgcn_perm(vb.x, va.x, 0x07060302u),
                __builtin_amdgcn_perm(vb.y, va.y, 0x05040100u), __builtin_amdgcn_perm(vb.y, va.y, 0x07060302u),
                __builtin_amdgcn_perm(vb.z, va.z, 0x05040100u), __builtin_amdgcn_perm(vb.z, va.z, 0x07060302u),
                __builtin_amdgcn_perm(vb.w, va.w, 0x05040100u), __builtin_amdgcn_perm(vb.w, va.w, 0x07060302u)};
            uint32_t pp[GM];
#pragma unroll
            for (int g4 = 0; g4 < GM / 4; ++g4) {
                const float4 pa = *reinterpret_cast<const float4*>(&sm.p[wave][ka][4 * g4]);
                const float4 pb = *reinterpret_cast<const float4*>(&sm.p[wave][kb][4 * g4]);
                pp[4 * g4] = pack_bf16x2(pa.x, pb.x);
                pp[4 * g4 + 1] = pack_bf16x2(pa.y, pb.y);
                pp[4 * g4 + 2] = pack_bf16x2(pa.z, pb.z);
                pp[4 * g4 + 3] = pack_bf16x2(pa.w, pb.w);
            }
#pragma unroll
            for (int g = 0; g < GM; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] = dot2_bf16(pp[g], vp[e], acc[g][e]);
        }
    }

    // wavefront state: sums over the 4 lanes of a head, numerators over the 4 key phases
    l_run += __shfl_xor(l_run, 16, kWave);
    l_run += __shfl_xor(l_run, 32, kWave);
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[g][e] += __shfl_xor(acc[g][e], 16, kWave);
            acc[g][e] += __shfl_xor(acc[g][e], 32, kWave);
        }
    if (r4 == 0) {
        sm.m[wave][r16] = m_run;
        sm.l[wave][r16] = l_run;
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.acc[wave][g][8 * r16 + e] = acc[g][e];
    }
    __syncthreads();

    // merge the four wavefronts (a wavefront without blocks has m = -inf, l = 0)
    const size_t idx = (size_t)kvh * a.nsplit + blockIdx.x;
    for (int i = threadIdx.x; i < G * kAttnD; i += blockDim.x) {
        const int g = i / kAttnD, d = i - g * kAttnD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm.m[w][g]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float sw = exp2f((sm.m[w][g] - M) * a.c);
            num = fmaf(sm.acc[w][g][d], sw, num);
            den = fmaf(sm.l[w][g], sw, den);
        }
        a.part_a[(idx * GM + g) * kAttnD + d] = num;
        if (d == 0) {
            a.part_m[idx * kAttnHeads + g] = M;
            a.part_l[idx * kAttnHeads + g] = den;
        }
    }
}

// One query head, 16 columns of d per workgroup; thread (phase, column) takes
// every 16th split.  Two passes over the loaded values: the maximum, then the
// rescaled sums.
constexpr int kCmbPhases = 16;
constexpr int kCmbMaxPer = kAttnMaxSplits / kCmbPhases;

template <int GM>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
    __shared__ float s_red[kCmbPhases][16];
    __shared__ float s_den[kCmbPhases];
    const int h = blockIdx.x;
    const int kvh = h / a.G, g = h - kvh * a.G;
    const int col = threadIdx.x & 15, ph = threadIdx.x >> 4;
    const int d = 16 * blockIdx.y + col;
    float mv[kCmbMaxPer], lv[kCmbMaxPer], av[kCmbMaxPer];
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kCmbMaxPer; ++j) {
        const int s = ph + kCmbPhases * j;
        mv[j] = -INFINITY;
        lv[j] = 0.f;
        av[j] = 0.f;
        if (s < a.nsplit) {
            const size_t idx = (size_t)kvh * a.nsplit + s;
            mv[j] = a.part_m[idx * kAttnHeads + g];
            lv[j] = a.part_l[idx * kAttnHeads + g];
            av[j] = a.part_a[(idx * GM + g) * kAttnD + d];
        }
        M = fmaxf(M, mv[j]);
    }
    s_red[ph][col] = M;
    __syncthreads();
    M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCmbPhases; ++i) M = fmaxf(M, s_red[i][col]);   // every split has a block
    __syncthreads();
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int j = 0; j < kCmbMaxPer; ++j) {
        const float w = exp2f((mv[j] - M) * a.c);
        num = fmaf(av[j], w, num);
        den = fmaf(lv[j], w, den);
    }
    s_red[ph][col] = num;
    if (col == 0) s_den[ph] = den;
    __syncthreads();
    if (ph == 0) {
        float n = 0.f, z = 0.f;
#pragma unroll
        for (int i = 0; i < kCmbPhases; ++i) {
            n += s_red[i][col];
            z += s_den[i];
        }
        a.out[(size_t)h * kAttnD + d] = (uint16_t)f32_to_bf16(n / z);
    }
}

template <int GM>
static hipError_t attn_gm(const AttnArgs& a, hipStream_t st, KernelTimer& tm) {
    tm.before();
    tm.launch(k_attn_split<GM>, dim3(a.nsplit, a.Hkv), dim3(256), 0, st, a);
    tm.after();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    tm.launch(k_attn_combine<GM>, dim3(a.Hkv * a.G, kAttnD / 16), dim3(256), 0, st, a);
    tm.after();
    return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t st, KernelTimer& tm) {
    return a.G <= 8 ? attn_gm<8>(a, st, tm) : attn_gm<16>(a, st, tm);
}

}  // namespace moe_w4
