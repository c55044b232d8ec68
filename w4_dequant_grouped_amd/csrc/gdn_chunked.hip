// Gated DeltaNet scan in chunks of 64 tokens on bf16 MFMA, gfx950.
//
// The same recurrence as k_gdn_scan (the published gated delta rule, per value
// head h over query/key head h / rep; "Perplexity built an inference engine for
// one model, one chip", paragraph 2: the model's linear-attention layers keep a
// fixed-size state):
//     S_t = a_t S_{t-1} + beta_t (v_t - a_t S_{t-1} k_t) k_t^T,   o_t = S_t q_t
// rewritten per chunk so that everything except a 64 x 64 triangular inverse is
// a matrix product.  Within a chunk (positions t, s = 0..63), with G_t the
// running sum of the log decays g and gamma_t = exp(G_t):
//     u_t := beta_t (v_t - a_t S_{t-1} k_t)   satisfies   (I + A) U = diag(beta) (V - Gamma K S_0^T)
//     A[t][s] = beta_t exp(G_t - G_s) k_t.k_s   (s < t)
// so with Tinv = (I + A)^-1, Tb = Tinv diag(beta), Tbg = Tinv diag(beta gamma):
//     U   = Vt - W S_0^T,              Vt = Tb V,  W = Tbg K
//     O   = Gamma Q S_0^T + Pm U,      Pm[t][s] = exp(G_t - G_s) q_t.k_s   (s <= t)
//     S_C = gamma_63 S_0 + U^T diag(d) K,   d_s = exp(G_63 - G_s)
// (all decays appear as exp of a non-positive difference, never as a ratio).
//
// k_gdn_prep: one workgroup per (chunk, value head), every chunk at once.  K K^T
//   and K Q^T on MFMA; the masks and decays; Tinv in three levels (four 16 x 16
//   diagonal blocks by forward substitution in fp32, then the 16- and 32-wide
//   off-diagonal blocks as products of inverses); W^T = K^T Tbg^T and Vt = Tb V
//   on MFMA.  Everything the sequential scan needs is written to the workspace
//   already in the lane layout of its MFMA operands.
// k_gdn_chunk_scan: one workgroup per (16 value rows, value head), chunk after
//   chunk, two barriers per chunk.  The state is held as S^T in the layout of an
//   MFMA result (lane l: key rows 4(l/16)..+3 of a 16-key block, value row
//   l%16); two such blocks side by side are exactly a 32-deep B operand, so the
//   state, U and d U feed the next products straight from registers or LDS.
//
// MFMA: v_mfma_f32_16x16x32_bf16, lane l holding A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] and C[4(l/16)+r][l%16].  Operands that the scan builds from
// two result blocks use the contraction order "paired blocks": slot e of lane
// group g is index 4g+e of the first 16-block for e < 4 and index 16+4g+(e-4) of
// the second; the workspace fragments that meet them are written in that same
// order.  fp32 operands enter as bf16 hi + lo pairs: hi*hi + hi*lo + lo*hi when
// both sides are split, hi*x + lo*x against exact bf16 data (q, k, v).
#include "device.h"
#include "kernels.h"

namespace moe_w4 {

namespace {

constexpr int kC = 64;            // tokens per chunk
constexpr int kD = 128;           // head dimension
constexpr int kRB = 16;           // value rows per scan wavefront
constexpr int kSub = 1;           // value-row blocks per scan workgroup (four wavefronts each)
constexpr int kAhead = 2;         // chunks between an operand load and its use

// Workspace, in 4-byte words.  Per (chunk, value head):
//   -W  fragments [token block 4][key group 4]    2048 B each: 64 lanes x 16 B hi, then lo
//   Pm  fragments [token block 4][token group 2]  same format (group 1 only for blocks 2, 3)
//   Vt  fragments [token block 4][value block 8]  64 lanes x 4 floats, result layout
//   gamma [64], d [64]
// then per (chunk, key head): K^T fragments [key block 8][token group 2] and Q
// fragments [token block 4][key group 4], 64 lanes x 8 bf16 each.
constexpr int kFragSplit = 512;                       // words of a split fragment
constexpr int kOffW = 0;
constexpr int kOffP = kOffW + 16 * kFragSplit;
constexpr int kOffV = kOffP + 8 * kFragSplit;
constexpr int kOffG = kOffV + 32 * 256;
constexpr int kHeadWords = kOffG + 2 * kC;            // 20608
constexpr int kOffQ = 16 * 256;                       // Q fragments within a key block
constexpr int kKeyWords = 2 * 16 * 256;               // 8192

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// x = hi + lo, hi = bf16(x), lo = bf16(x - hi); four values -> two dwords each
struct Half4 {
    u32x2 hi, lo;
};
__device__ __forceinline__ Half4 split4(const f32x4& x) {
    const uint32_t h01 = pack_bf16x2(x[0], x[1]), h23 = pack_bf16x2(x[2], x[3]);
    Half4 r;
    r.hi = u32x2{h01, h23};
    r.lo = u32x2{pack_bf16x2(x[0] - bf16lo(h01), x[1] - bf16hi(h01)),
                 pack_bf16x2(x[2] - bf16lo(h23), x[3] - bf16hi(h23))};
    return r;
}
// eight values (a: slots 0..3, b: slots 4..7) as one split 32-deep operand
struct Split8 {
    u32x4 hi, lo;
};
__device__ __forceinline__ Split8 split8(const f32x4& a, const f32x4& b) {
    const Half4 x = split4(a), y = split4(b);
    return Split8{u32x4{x.hi.x, x.hi.y, y.hi.x, y.hi.y}, u32x4{x.lo.x, x.lo.y, y.lo.x, y.lo.y}};
}
__device__ __forceinline__ u32x4 cat(const u32x2& a, const u32x2& b) { return u32x4{a.x, a.y, b.x, b.y}; }

// 16 x 16 x 16 product of split fp32 operands (the inverse's off-diagonal blocks)
__device__ __forceinline__ f32x4 mma3_16(const Half4& a, const Half4& b, f32x4 c) {
    const s16x4 ah = __builtin_bit_cast(s16x4, a.hi), al = __builtin_bit_cast(s16x4, a.lo);
    const s16x4 bh = __builtin_bit_cast(s16x4, b.hi), bl = __builtin_bit_cast(s16x4, b.lo);
    c = mfma16(ah, bh, c);
    c = mfma16(ah, bl, c);
    return mfma16(al, bh, c);
}

// A operand (rows m0 + l%16, columns k0 + 4 (l/16) ..) and B operand (rows
// k0 + 4 (l/16) .., column n0 + l%16) of a 16 x 16 x 16 product, from a row-major
// fp32 LDS matrix
__device__ __forceinline__ Half4 lds_a16(const float (*m)[kC + 4], int m0, int k0, int lane) {
    const float4 v = *reinterpret_cast<const float4*>(&m[m0 + (lane & 15)][k0 + 4 * (lane >> 4)]);
    return split4(f32x4{v.x, v.y, v.z, v.w});
}
__device__ __forceinline__ Half4 lds_b16(const float (*m)[kC + 4], int k0, int n0, int lane) {
    const int k = k0 + 4 * (lane >> 4), n = n0 + (lane & 15);
    return split4(f32x4{m[k][n], m[k + 1][n], m[k + 2][n], m[k + 3][n]});
}

// 4 tokens x 4 columns of bf16 (rows r[0..3], two dwords each) -> 4 columns x 4 tokens
__device__ __forceinline__ void transpose4(const u32x2 (&r)[4], u32x2 (&c)[4]) {
    c[0] = u32x2{(r[0].x & 0xFFFFu) | (r[1].x << 16), (r[2].x & 0xFFFFu) | (r[3].x << 16)};
    c[1] = u32x2{(r[0].x >> 16) | (r[1].x & 0xFFFF0000u), (r[2].x >> 16) | (r[3].x & 0xFFFF0000u)};
    c[2] = u32x2{(r[0].y & 0xFFFFu) | (r[1].y << 16), (r[2].y & 0xFFFFu) | (r[3].y << 16)};
    c[3] = u32x2{(r[0].y >> 16) | (r[1].y & 0xFFFF0000u), (r[2].y >> 16) | (r[3].y & 0xFFFF0000u)};
}

__device__ __forceinline__ float* head_block(const GdnChunkArgs& a, int c, int h) {
    return a.ws + ((size_t)c * a.Hv + h) * kHeadWords;
}
__device__ __forceinline__ float* key_block(const GdnChunkArgs& a, int nch, int c, int kh) {
    return a.ws + (size_t)nch * a.Hv * kHeadWords + ((size_t)c * a.Hk + kh) * kKeyWords;
}

}  // namespace

// ---------------------------------------------------------------------------
// k_gdn_prep
// ---------------------------------------------------------------------------
// At most 128 registers (four workgroups per CU; two values spill to scratch), so
// that the 1024 workgroups of a 2048-token segment are resident in one round: at
// 160 registers three fitted, and the second round's workgroups started only
// when the first finished (30.3 -> 26.0 us at 2048 tokens, 32 value heads).
__global__ __launch_bounds__(256, 4) void k_gdn_prep(GdnChunkArgs a) {
    // Two LDS regions, each reused across the phases, so that four workgroups fit
    // a CU and a segment's workgroups are resident together:
    //   region 1: K rows [64][136] bf16 -> A, then Tinv, [64][68] fp32 -> V^T [128][72] bf16
    //   region 2: Q rows [64][136] bf16 -> K^T [128][72] bf16
    constexpr int kRegion = kD * (kC + 8) * 2;                               // the largest use, 18 KiB
    __shared__ __attribute__((aligned(16))) unsigned char s_r1[kRegion], s_r2[kRegion];
    __shared__ __attribute__((aligned(16))) float s_g[kC], s_b[kC], s_bg[kC];   // s_g: G log2(e)
    uint16_t (*s_k)[kD + 8] = reinterpret_cast<uint16_t (*)[kD + 8]>(s_r1);
    float (*s_a)[kC + 4] = reinterpret_cast<float (*)[kC + 4]>(s_r1);
    uint16_t (*s_vt)[kC + 8] = reinterpret_cast<uint16_t (*)[kC + 8]>(s_r1);
    uint16_t (*s_q)[kD + 8] = reinterpret_cast<uint16_t (*)[kD + 8]>(s_r2);
    uint16_t (*s_kt)[kC + 8] = reinterpret_cast<uint16_t (*)[kC + 8]>(s_r2);
    static_assert(sizeof(uint16_t) * kC * (kD + 8) <= kRegion && sizeof(float) * kC * (kC + 4) <= kRegion,
                  "LDS regions");

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g4 = lane >> 4, ln = lane & 15;
    const int c = blockIdx.x, h = blockIdx.y;
    const int kh = h / a.rep;
    const int nch = (a.nt + kC - 1) / kC;
    const int t0 = a.t0 + c * kC;
    const int nt = min(kC, a.t0 + a.nt - t0);
    float* hb = head_block(a, c, h);

    // decays and write strengths; tokens past the sequence have g = 0, beta = 0
    if (wave == 0) {
        const bool ok = lane < nt;
        const size_t gi = (size_t)(t0 + lane) * a.Hv + h;
        float gv = ok ? a.g[gi] : 0.f;
        const float bv = ok ? a.beta[gi] : 0.f;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const float v = __shfl_up(gv, o, kWave);
            if (lane >= o) gv += v;
        }
        // decays as 2^(G log2 e) on the hardware exp2 (about one ulp, as expf)
        const float g2 = gv * 1.4426950408889634f;
        const float gam = __builtin_amdgcn_exp2f(g2);
        s_g[lane] = g2;
        s_b[lane] = bv;
        s_bg[lane] = bv * gam;
        hb[kOffG + lane] = gam;
        hb[kOffG + kC + lane] = __builtin_amdgcn_exp2f(__shfl(g2, kC - 1, kWave) - g2);
    }
    // K, Q and V of the chunk (zero past the sequence): each thread one unit of
    // tokens 4 tq .. +3 and columns 8 cg .. +7, loaded once.  K and Q rows go to
    // LDS; K^T and V^T wait in registers for their regions.
    const int tq = threadIdx.x & 15, cg = threadIdx.x >> 4;
    u32x2 ktile[8], vtile[8];
    {
        u32x4 kr[4], qr[4], vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * tq + r;
            const bool ok = t < nt;
            const size_t ko = ((size_t)(t0 + t) * a.Hk + kh) * kD + 8 * cg;
            kr[r] = ok ? load_u32x4(a.k + ko) : u32x4{0u, 0u, 0u, 0u};
            qr[r] = ok ? load_u32x4(a.q + ko) : u32x4{0u, 0u, 0u, 0u};
            vr[r] = ok ? load_u32x4(a.v + ((size_t)(t0 + t) * a.Hv + h) * kD + 8 * cg) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *reinterpret_cast<u32x4*>(&s_k[4 * tq + r][8 * cg]) = kr[r];
            *reinterpret_cast<u32x4*>(&s_q[4 * tq + r][8 * cg]) = qr[r];
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {          // columns 8 cg + 4 hf .. + 3
            const u32x2 kh2[4] = {u32x2{kr[0][2 * hf], kr[0][2 * hf + 1]}, u32x2{kr[1][2 * hf], kr[1][2 * hf + 1]},
                                  u32x2{kr[2][2 * hf], kr[2][2 * hf + 1]}, u32x2{kr[3][2 * hf], kr[3][2 * hf + 1]}};
            const u32x2 vh2[4] = {u32x2{vr[0][2 * hf], vr[0][2 * hf + 1]}, u32x2{vr[1][2 * hf], vr[1][2 * hf + 1]},
                                  u32x2{vr[2][2 * hf], vr[2][2 * hf + 1]}, u32x2{vr[3][2 * hf], vr[3][2 * hf + 1]}};
            u32x2 kc[4], vc[4];
            transpose4(kh2, kc);
            transpose4(vh2, vc);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                ktile[4 * hf + d] = kc[d];
                vtile[4 * hf + d] = vc[d];
            }
        }
    }
    __syncthreads();

    // Q fragments of the scan's Q S^T (token block = wave, key group p), paired-
    // block order, once per key head
    if (h % a.rep == 0) {
        u32x4* qf = reinterpret_cast<u32x4*>(key_block(a, nch, c, kh) + kOffQ);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint16_t* row = &s_q[16 * wave + ln][32 * p + 4 * g4];
            qf[(wave * 4 + p) * 64 + lane] = cat(*reinterpret_cast<const u32x2*>(row),
                                                 *reinterpret_cast<const u32x2*>(row + 16));
        }
    }

    // K K^T and K Q^T as transposed blocks [s block sb][t block = wave]: lane holds
    // s = 16 sb + 4 g4 + r, t = 16 wave + ln.  A (strictly lower, times beta_t) and
    // Pm stay in registers until K's and Q's regions are free.
    f32x4 pm[4], am[4];
    {
        const int t = 16 * wave + ln;
        const float gt = s_g[t], bt = s_b[t];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            f32x4 kk = {0.f, 0.f, 0.f, 0.f}, kq = kk;
            if (sb <= wave) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const u32x4 as = *reinterpret_cast<const u32x4*>(&s_k[16 * sb + ln][32 * p + 8 * g4]);
                    const u32x4 bk = *reinterpret_cast<const u32x4*>(&s_k[t][32 * p + 8 * g4]);
                    const u32x4 bq = *reinterpret_cast<const u32x4*>(&s_q[t][32 * p + 8 * g4]);
                    kk = mfma32(as, bk, kk);
                    kq = mfma32(as, bq, kq);
                }
            }
            f32x4 av, pv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * sb + 4 * g4 + r;
                const float dec = (s <= t) ? __builtin_amdgcn_exp2f(gt - s_g[s]) : 0.f;
                av[r] = (s < t) ? bt * dec * kk[r] : 0.f;
                pv[r] = dec * kq[r];
            }
            pm[sb] = pv;
            am[sb] = av;
        }
    }
    // Pm fragments [token block wave][token group p]
    {
        float* pf = hb + kOffP;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (2 * p > wave) continue;
            const Split8 sp = split8(pm[2 * p], pm[2 * p + 1]);
            u32x4* f = reinterpret_cast<u32x4*>(pf + (wave * 2 + p) * kFragSplit);
            f[lane] = sp.hi;
            f[64 + lane] = sp.lo;
        }
    }
    __syncthreads();          // K and Q rows no longer read: A and K^T take their regions
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
        *reinterpret_cast<f32x4*>(&s_a[16 * wave + ln][16 * sb + 4 * g4]) = am[sb];
#pragma unroll
    for (int d = 0; d < 8; ++d) *reinterpret_cast<u32x2*>(&s_kt[8 * cg + d][4 * tq]) = ktile[d];
    __syncthreads();

    // K^T fragments of the scan's state update (key block jb, token group p),
    // paired-block order, once per key head
    if (h % a.rep == 0) {
        u32x4* kf = reinterpret_cast<u32x4*>(key_block(a, nch, c, kh));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int jb = 2 * wave + i;
                const uint16_t* row = &s_kt[16 * jb + ln][32 * p + 4 * g4];
                kf[(jb * 2 + p) * 64 + lane] = cat(*reinterpret_cast<const u32x2*>(row),
                                                   *reinterpret_cast<const u32x2*>(row + 16));
            }
    }

    // Tinv level 1: wavefront w inverts its diagonal block I + A_ww by forward
    // substitution in fp32, lane c < 16 holding column c
    if (lane < 16) {
        const int o = 16 * wave;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc0 = (t == lane) ? 1.f : 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll
            for (int s = 0; s < t; s += 4) {
                const float4 av = *reinterpret_cast<const float4*>(&s_a[o + t][o + s]);
                acc0 = fmaf(-av.x, x[s], acc0);
                if (s + 1 < t) acc1 = fmaf(-av.y, x[s + 1], acc1);
                if (s + 2 < t) acc2 = fmaf(-av.z, x[s + 2], acc2);
                if (s + 3 < t) acc3 = fmaf(-av.w, x[s + 3], acc3);
            }
            x[t] = (acc0 + acc1) + (acc2 + acc3);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) s_a[o + t][o + lane] = x[t];
    }
    __syncthreads();

    // level 2: X_10 = -X_11 A_10 X_00 (wavefront 0), X_32 = -X_33 A_32 X_22 (wavefront 2)
    if (wave == 0 || wave == 2) {
        const int i = wave + 1, j = wave;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 r = mma3_16(lds_a16(s_a, 16 * i, 16 * j, lane), lds_b16(s_a, 16 * j, 16 * j, lane), z);
        const f32x4 x = mma3_16(lds_a16(s_a, 16 * i, 16 * i, lane), split4(r), z);
#pragma unroll
        for (int e = 0; e < 4; ++e) s_a[16 * i + 4 * g4 + e][16 * j + ln] = -x[e];
    }
    __syncthreads();

    // level 3: the 32 x 32 block below the diagonal, X_ij for i = 2, 3 and j = 0, 1:
    // Y_kj = sum_{m = 0, 1} A_km X_mj, X_ij = -sum_{k = 2..i} X_ik Y_kj
    {
        const int i = 2 + (wave >> 1), j = wave & 1;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 y2 = mma3_16(lds_a16(s_a, 32, 16, lane), lds_b16(s_a, 16, 16 * j, lane), z);
        if (j == 0) y2 = mma3_16(lds_a16(s_a, 32, 0, lane), lds_b16(s_a, 0, 0, lane), y2);
        f32x4 x = mma3_16(lds_a16(s_a, 16 * i, 32, lane), split4(y2), z);
        if (i == 3) {
            f32x4 y3 = mma3_16(lds_a16(s_a, 48, 16, lane), lds_b16(s_a, 16, 16 * j, lane), z);
            if (j == 0) y3 = mma3_16(lds_a16(s_a, 48, 0, lane), lds_b16(s_a, 0, 0, lane), y3);
            x = mma3_16(lds_a16(s_a, 48, 48, lane), split4(y3), x);
        }
        __syncthreads();      // every read of A_2j, A_3j done before they are overwritten
#pragma unroll
        for (int e = 0; e < 4; ++e) s_a[16 * i + 4 * g4 + e][16 * j + ln] = -x[e];
    }
    __syncthreads();          // Tinv complete (zero above the diagonal)

    // rows t = 16 wave + ln of Tb and Tbg over token groups p (natural order);
    // Tinv is zero for s > t, so blocks 0 and 1 need group 0 only
    const int np = wave >= 2 ? 2 : 1;
    Split8 tbs[2], tgs[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (p >= np) continue;
        const int s0 = 32 * p + 8 * g4;
        const float* row = &s_a[16 * wave + ln][s0];
        const float4 x0 = *reinterpret_cast<const float4*>(row), x1 = *reinterpret_cast<const float4*>(row + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(&s_b[s0]), b1 = *reinterpret_cast<const float4*>(&s_b[s0 + 4]);
        const float4 c0 = *reinterpret_cast<const float4*>(&s_bg[s0]), c1 = *reinterpret_cast<const float4*>(&s_bg[s0 + 4]);
        tbs[p] = split8(f32x4{x0.x * b0.x, x0.y * b0.y, x0.z * b0.z, x0.w * b0.w},
                        f32x4{x1.x * b1.x, x1.y * b1.y, x1.z * b1.z, x1.w * b1.w});
        tgs[p] = split8(f32x4{x0.x * c0.x, x0.y * c0.y, x0.z * c0.z, x0.w * c0.w},
                        f32x4{x1.x * c1.x, x1.y * c1.y, x1.z * c1.z, x1.w * c1.w});
    }
    __syncthreads();          // Tinv no longer read: V^T takes its region
#pragma unroll
    for (int d = 0; d < 8; ++d) *reinterpret_cast<u32x2*>(&s_vt[8 * cg + d][4 * tq]) = vtile[d];
    __syncthreads();

    // W^T = K^T Tbg^T as blocks [key block jb][token block wave]: lane holds
    // W[16 wave + ln][16 jb + 4 g4 + r], two blocks = one -W fragment (paired order)
    {
        u32x4* wf = reinterpret_cast<u32x4*>(hb + kOffW);
#pragma unroll
        for (int pk = 0; pk < 4; ++pk) {
            f32x4 w2[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int jb = 2 * pk + i;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    if (p >= np) continue;
                    const u32x4 ak = *reinterpret_cast<const u32x4*>(&s_kt[16 * jb + ln][32 * p + 8 * g4]);
                    acc = mfma32(ak, tgs[p].hi, acc);
                    acc = mfma32(ak, tgs[p].lo, acc);
                }
                w2[i] = -acc;
            }
            const Split8 sp = split8(w2[0], w2[1]);
            wf[(wave * 4 + pk) * 128 + lane] = sp.hi;
            wf[(wave * 4 + pk) * 128 + 64 + lane] = sp.lo;
        }
    }
    // Vt = Tb V as blocks [token block wave][value block vb], stored in result layout
    {
        f32x4* vf = reinterpret_cast<f32x4*>(hb + kOffV);
#pragma unroll
        for (int vb = 0; vb < 8; ++vb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                if (p >= np) continue;
                const u32x4 bv = *reinterpret_cast<const u32x4*>(&s_vt[16 * vb + ln][32 * p + 8 * g4]);
                acc = mfma32(tbs[p].hi, bv, acc);
                acc = mfma32(tbs[p].lo, bv, acc);
            }
            vf[(wave * 8 + vb) * 64 + lane] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// k_gdn_chunk_scan
// ---------------------------------------------------------------------------
namespace {
// Operands of one chunk for one wavefront (token block = wave; key blocks
// 2 wave, 2 wave + 1), loaded kAhead chunks ahead so that their memory latency
// (the prep kernel's output, mostly out of the L2) overlaps the work between.
struct ScanOps {
    u32x4 wh[4], wl[4];      // -W fragments, key groups 0..3
    u32x4 ph[2], pl[2];      // Pm fragments, token groups 0, 1 (group 1: blocks 2, 3 only)
    u32x4 q[4];              // Q row 16 wave + l%16, key groups 0..3, paired order
    u32x4 kt[2][2];          // K^T fragments [key block 2 wave + i][token group]
    f32x4 vt;                // Vt block [wave][value block]
    f32x4 gam, dec;          // gamma_t and d_t of rows 16 wave + 4 (l/16) .. + 3
    float gend;              // gamma_63
};

// Buffer resources of the segment and this lane's fixed byte offsets.  Chunk-
// dependent parts of workspace addresses go to the scalar offset.  The output
// keeps the whole offset in the lane's register, which the range check covers: a
// raw buffer store at or past num_records stores nothing, and that drops the
// rows past the sequence in the last chunk.
struct ScanMem {
    __amdgpu_buffer_rsrc_t ws, out;
    const float* wsp;                    // the workspace again, for the one scalar read
    int vw, vp, vq, vk, vv, vg;          // -W, Pm, Q, K^T, Vt, gamma
    int vo[4];                           // output rows 16 wave + 4 (l/16) + r
    int head_base;                       // this head's block within a chunk (the lane offsets include it)
    int head_stride, key_base, key_stride, o_stride;   // bytes
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, int v, int s) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0);
}
__device__ __forceinline__ u32x2 ld8(__amdgpu_buffer_rsrc_t r, int v, int s) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, v, s, 0);
}

// Loads of one chunk's operands in pieces; the scan issues them in three groups,
// one per phase of a chunk.
__device__ __forceinline__ void load_w(ScanOps& o, const ScanMem& m, int c, int p) {
    const int off = c * m.head_stride + 4 * kOffW + 2048 * p;
    o.wh[p] = ld16(m.ws, m.vw, off);
    o.wl[p] = ld16(m.ws, m.vw + 1024, off);
}
__device__ __forceinline__ void load_q(ScanOps& o, const ScanMem& m, int c, int p) {
    o.q[p] = ld16(m.ws, m.vq, m.key_base + c * m.key_stride + 4 * kOffQ + 1024 * p);
}
__device__ __forceinline__ void load_pm(ScanOps& o, const ScanMem& m, int c, int p) {
    const int off = c * m.head_stride + 4 * kOffP + 2048 * p;
    o.ph[p] = ld16(m.ws, m.vp, off);
    o.pl[p] = ld16(m.ws, m.vp + 1024, off);
}
__device__ __forceinline__ void load_kt(ScanOps& o, const ScanMem& m, int c, int i) {
    const int off = m.key_base + c * m.key_stride + 2048 * i;
    o.kt[i][0] = ld16(m.ws, m.vk, off);
    o.kt[i][1] = ld16(m.ws, m.vk, off + 1024);
}
__device__ __forceinline__ void load_misc(ScanOps& o, const ScanMem& m, int c) {
    const int hoff = c * m.head_stride;
    o.vt = __builtin_bit_cast(f32x4, ld16(m.ws, m.vv, hoff + 4 * kOffV));
    o.gam = __builtin_bit_cast(f32x4, ld16(m.ws, m.vg, hoff + 4 * kOffG));
    o.dec = __builtin_bit_cast(f32x4, ld16(m.ws, m.vg, hoff + 4 * (kOffG + kC)));
    // gamma_63 is the same for every lane: a scalar read, outside the vector
    // memory counter (two chunks of vector loads already fill most of its range)
    o.gend = m.wsp[(m.head_base + hoff) / 4 + kOffG + kC - 1];
}
__device__ __forceinline__ void load_ops(ScanOps& o, const ScanMem& m, int c) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        load_w(o, m, c, p);
        load_q(o, m, c, p);
    }
    load_pm(o, m, c, 0);
    load_pm(o, m, c, 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) load_kt(o, m, c, i);
    load_misc(o, m, c);
}
}  // namespace

// Wavefront w + 4 sub takes token block w (and key blocks 2w, 2w + 1) of
// value-row block kSub (workgroup / Hv) + sub.  One row block per workgroup
// measured fastest: the operand fetch of a CU is limited by the requests it can
// keep in flight, and a second row block doubles them without sharing them.
__global__ __launch_bounds__(256 * kSub) void k_gdn_chunk_scan(GdnChunkArgs a) {
    __shared__ __attribute__((aligned(16))) u32x4 s_sh[kSub][4][kWave], s_sl[kSub][4][kWave];   // S^T key groups, split
    __shared__ __attribute__((aligned(16))) u32x2 s_uh[kSub][4][kWave], s_ul[kSub][4][kWave];   // U blocks, split
    __shared__ __attribute__((aligned(16))) u32x2 s_dh[kSub][4][kWave], s_dl[kSub][4][kWave];   // d U blocks, split
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (threadIdx.x / kWave) & 3;
    const int sub = threadIdx.x / (4 * kWave);
    const int g4 = lane >> 4, ln = lane & 15;
    const int h = blockIdx.x % a.Hv;
    const int rb = kSub * (blockIdx.x / a.Hv) + sub;
    const int kh = h / a.rep;
    const int iv = kRB * rb + ln;                 // this lane's value row
    const int nch = (a.nt + kC - 1) / kC;
    float* state = a.state + ((size_t)h * kD + iv) * kD;

    ScanMem m;
    m.head_stride = a.Hv * kHeadWords * 4;
    m.key_stride = a.Hk * kKeyWords * 4;
    m.key_base = nch * m.head_stride + kh * kKeyWords * 4;
    m.o_stride = a.Hv * kD * 2;
    m.ws = make_rsrc(a.ws, (uint32_t)nch * (uint32_t)(m.head_stride + m.key_stride));
    m.wsp = a.ws;
    m.out = make_rsrc(a.out + (size_t)a.t0 * a.Hv * kD, (uint32_t)a.nt * m.o_stride);
    const int hb0 = h * kHeadWords * 4;
    m.head_base = hb0;
    m.vw = hb0 + (wave * 4 * 128 + lane) * 16;
    m.vp = hb0 + (wave * 2 * 128 + lane) * 16;
    m.vq = (4 * wave * 64 + lane) * 16;
    m.vk = (4 * wave * 64 + lane) * 16;
    m.vv = hb0 + ((wave * 8 + rb) * 64 + lane) * 16;
    m.vg = hb0 + (16 * wave + 4 * g4) * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) m.vo[r] = (16 * wave + 4 * g4 + r) * m.o_stride + h * kD * 2 + 2 * iv;

    // S^T key blocks 2 wave, 2 wave + 1: lane holds S[iv][32 wave + 16 i + 4 g4 + r]
    f32x4 sm[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(state + 32 * wave + 16 * i + 4 * g4);
        sm[i] = f32x4{v.x, v.y, v.z, v.w};
    }
    auto publish = [&]() {        // this wavefront's key group as a split B operand
        const Split8 sp = split8(sm[0], sm[1]);
        s_sh[sub][wave][lane] = sp.hi;
        s_sl[sub][wave][lane] = sp.lo;
    };
    publish();

    auto step = [&](const ScanOps& cur, ScanOps& nxt, int c) {
        const int cn = min(c + kAhead, nch - 1);  // operands in flight for kAhead chunks
#pragma unroll
        for (int p = 0; p < 4; ++p) load_w(nxt, m, cn, p);
        __syncthreads();          // the state's key groups are current

        // U = Vt - W S^T and QS = Q S^T for token block `wave`
        f32x4 u = cur.vt, qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4 sh = s_sh[sub][p][lane], sl = s_sl[sub][p][lane];
            u = mfma32(cur.wh[p], sh, u);
            qs = mfma32(cur.q[p], sh, qs);
            u = mfma32(cur.wh[p], sl, u);
            qs = mfma32(cur.q[p], sl, qs);
            u = mfma32(cur.wl[p], sh, u);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) load_q(nxt, m, cn, p);
        // (token group 1 of Pm is used, and written, for token blocks 2, 3 only;
        // the other wavefronts load it too, as a conditional load would make
        // the compiler's waits on the memory counter conservative)
        load_pm(nxt, m, cn, 0);
        load_pm(nxt, m, cn, 1);
        const Half4 us = split4(u), ds = split4(u * cur.dec);
        s_uh[sub][wave][lane] = us.hi;
        s_ul[sub][wave][lane] = us.lo;
        s_dh[sub][wave][lane] = ds.hi;
        s_dl[sub][wave][lane] = ds.lo;
        __syncthreads();          // every U block written; every key group read
#pragma unroll
        for (int i = 0; i < 2; ++i) load_kt(nxt, m, cn, i);
        load_misc(nxt, m, cn);

        // O = Gamma QS + Pm U over token groups p <= wave / 2, and
        // S^T <- gamma_63 S^T + K^T diag(d) U on key blocks 2 wave, 2 wave + 1
        f32x4 o = cur.gam * qs, s0 = cur.gend * sm[0], s1 = cur.gend * sm[1];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const u32x4 dh = cat(s_dh[sub][2 * p][lane], s_dh[sub][2 * p + 1][lane]);
            const u32x4 dl = cat(s_dl[sub][2 * p][lane], s_dl[sub][2 * p + 1][lane]);
            s0 = mfma32(cur.kt[0][p], dh, s0);
            s1 = mfma32(cur.kt[1][p], dh, s1);
            s0 = mfma32(cur.kt[0][p], dl, s0);
            s1 = mfma32(cur.kt[1][p], dl, s1);
            if (2 * p <= wave) {
                const u32x4 uh = cat(s_uh[sub][2 * p][lane], s_uh[sub][2 * p + 1][lane]);
                const u32x4 ul = cat(s_ul[sub][2 * p][lane], s_ul[sub][2 * p + 1][lane]);
                o = mfma32(cur.ph[p], uh, o);
                o = mfma32(cur.ph[p], ul, o);
                o = mfma32(cur.pl[p], uh, o);
            }
        }
        sm[0] = s0;
        sm[1] = s1;
        publish();                // read after the next chunk's first barrier
        const int ooff = c * kC * m.o_stride;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16(o[r]), m.out, m.vo[r] + ooff, 0, 0);
    };

    // kAhead + 1 operand sets in rotation; the loop body has no conditional step,
    // so every wait on the memory counter it compiles to is exact
    int c = 0;
    if constexpr (kAhead == 1) {
        ScanOps A, B;
        load_ops(A, m, 0);
        for (; c + 2 <= nch; c += 2) {
            step(A, B, c);
            step(B, A, c + 1);
        }
        if (c < nch) step(A, B, c);
    } else {
        ScanOps A, B, C;
        load_ops(A, m, 0);
        load_ops(B, m, min(1, nch - 1));
        // Drain the two chunks loaded here before the loop.  Without it the
        // compiler merges this path's pending loads into the loop header and
        // waits there for nearly every load of the previous chunk on each pass.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        for (; c + 3 <= nch; c += 3) {
            step(A, C, c);
            step(B, A, c + 1);
            step(C, B, c + 2);
        }
        if (c < nch) step(A, C, c);
        if (c + 1 < nch) step(B, A, c + 1);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
        *reinterpret_cast<float4*>(state + 32 * wave + 16 * i + 4 * g4) = float4{sm[i][0], sm[i][1], sm[i][2], sm[i][3]};
}

size_t gdn_chunked_workspace_floats(int T, int Hv, int Hk) {
    const int seg = T < kGdnSegT ? T : kGdnSegT;
    const size_t nch = (size_t)((seg + kC - 1) / kC);
    return nch * ((size_t)Hv * kHeadWords + (size_t)Hk * kKeyWords);
}

hipError_t launch_gdn_chunked(const GdnChunkArgs& base, hipStream_t st, KernelTimer& tm) {
    for (int t0 = 0; t0 < base.T; t0 += kGdnSegT) {
        GdnChunkArgs a = base;
        a.t0 = t0;
        a.nt = min(kGdnSegT, base.T - t0);
        const int nch = (a.nt + kC - 1) / kC;
        tm.before();
        tm.launch(k_gdn_prep, dim3(nch, a.Hv), dim3(256), 0, st, a);
        tm.after();
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        tm.before();
        tm.launch(k_gdn_chunk_scan, dim3(a.Hv * (kD / kRB / kSub)), dim3(256 * kSub), 0, st, a);
        tm.after();
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace moe_w4
