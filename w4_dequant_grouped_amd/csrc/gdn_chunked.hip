// Gated DeltaNet scan in chunks of 64 tokens on bf16 MFMA, gfx950.
//
// The same recurrence as k_gdn_scan (the published gated delta rule, per value
// head h over query/key head h / rep; "Perplexity built an inference engine for
// one model, one chip", paragraph 2: the model's linear-attention layers keep a
// fixed-size state):
//     S_t = a_t S_{t-1} + beta_t (v_t - a_t S_{t-1} k_t) k_t^T,   o_t = S_t q_t
// rewritten per chunk so that everything except a 64-step triangular solve is a
// matrix product.  Within a chunk (positions t, s = 0..63), with G_t the running
// sum of the log decays g and gamma_t = exp(G_t):
//     u_t := beta_t (v_t - a_t S_{t-1} k_t)   satisfies   (I + A) U = diag(beta) (V - Gamma K S_0^T)
//     A[t][s] = beta_t exp(G_t - G_s) k_t.k_s   (s < t)
// so with Tinv = (I + A)^-1, Tb = Tinv diag(beta), Tbg = Tinv diag(beta gamma):
//     U   = Tb V - W S_0^T,            W = Tbg K
//     O   = Gamma Q S_0^T + Pm U,      Pm[t][s] = exp(G_t - G_s) q_t.k_s   (s <= t)
//     S_C = gamma_63 S_0 + U^T diag(d) K,   d_s = exp(G_63 - G_s)
// (all decays appear as exp of a non-positive difference, never as a ratio).
//
// k_gdn_prep: one workgroup per (chunk, value head), all chunks at once: K K^T
//   and Q K^T on MFMA (bf16 inputs, exact products, fp32 sums), the decay masks,
//   Tinv by forward substitution (one wavefront, a column per lane, fp32), and W
//   = Tbg K on MFMA.  It stores W, Pm, Tb and the decays gamma and d in the workspace.
// k_gdn_chunk_scan: one workgroup per (16 value rows, value head), chunk after
//   chunk.  The state is held as S^T in the layout of a 16x16x16 MFMA result
//   (lane l: key columns 4(l/16)..+3 of a 16-column block, value row l%16), which
//   is also the layout of that MFMA's B operand, so the state, U and the outputs
//   feed the next products without transposes.  fp32 operands (the state, W, U,
//   Pm, Tb) enter the bf16 MFMA as hi + lo bf16 pairs: hi*hi + hi*lo + lo*hi when
//   both sides are split, hi*x + lo*x against exact bf16 data (q, k, v).
#include "device.h"
#include "kernels.h"

namespace moe_w4 {

namespace {

constexpr int kC = 64;            // tokens per chunk
constexpr int kD = 128;           // head dimension
constexpr int kRB = 16;           // value rows per scan workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// fp32 x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), four at a time
struct Split4 {
    s16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4(const f32x4& x) {
    Split4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t hb = f32_to_bf16(x[e]);
        r.hi[e] = (short)hb;
        r.lo[e] = (short)f32_to_bf16(x[e] - bf16_to_f32(hb));
    }
    return r;
}
__device__ __forceinline__ Split4 neg(const Split4& s) {
    Split4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r.hi[e] = (short)(s.hi[e] ^ (short)0x8000);
        r.lo[e] = (short)(s.lo[e] ^ (short)0x8000);
    }
    return r;
}
// a (split) times b (split): three bf16 products
__device__ __forceinline__ f32x4 mma3(const Split4& a, const Split4& b, f32x4 c) {
    c = mfma16(a.hi, b.hi, c);
    c = mfma16(a.hi, b.lo, c);
    return mfma16(a.lo, b.hi, c);
}
// a (split) times exact bf16 b, or exact a times split b
__device__ __forceinline__ f32x4 mma2(const Split4& a, const s16x4& b, f32x4 c) {
    c = mfma16(a.hi, b, c);
    return mfma16(a.lo, b, c);
}
__device__ __forceinline__ f32x4 mma2(const s16x4& a, const Split4& b, f32x4 c) {
    c = mfma16(a, b.hi, c);
    return mfma16(a, b.lo, c);
}

__device__ __forceinline__ s16x4 load_bf16x4(const uint16_t* p) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    return __builtin_bit_cast(s16x4, v);
}

}  // namespace

// Workspace of one (chunk, value head), 4-byte words: W [64][128], Pm [64][64] and
// Tb [64][64] as bf16 hi/lo pairs, grouped four columns at a time (eight bf16:
// the four hi, then the four lo, so one 16-byte load is an MFMA operand's split
// pair), then gamma [64] = exp(G_t) and d [64] = exp(G_63 - G_t), fp32.
constexpr size_t kGdnChunkFloats = (size_t)kC * kD + 2 * (size_t)kC * kC + 2 * kC;

namespace {
// Stores the split pair of x at column `col` of row `row` of a [rows][ncol] matrix
// in the grouped hi/lo format.
__device__ __forceinline__ void store_split(uint16_t* base, int ncol, int row, int col, float x) {
    const uint32_t hb = f32_to_bf16(x);
    const uint32_t lb = f32_to_bf16(x - bf16_to_f32(hb));
    uint16_t* g = base + ((size_t)row * (ncol / 4) + col / 4) * 8 + (col & 3);
    g[0] = (uint16_t)hb;
    g[4] = (uint16_t)lb;
}
__device__ __forceinline__ Split4 load_split(const uint16_t* base, int ncol, int row, int col4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + ((size_t)row * (ncol / 4) + col4 / 4) * 8);
    Split4 r;
    r.hi = __builtin_bit_cast(s16x4, u32x2{v.x, v.y});
    r.lo = __builtin_bit_cast(s16x4, u32x2{v.z, v.w});
    return r;
}
}  // namespace

// ---------------------------------------------------------------------------
// k_gdn_prep
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gdn_prep(GdnChunkArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_k[kC][kD + 8];    // K rows (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t s_q[kC][kD + 8];    // Q rows
    __shared__ __attribute__((aligned(16))) uint16_t s_kt[kD][kC + 8];   // K transposed
    __shared__ __attribute__((aligned(16))) float s_a[kC][kC + 4];       // A, then Tbg
    __shared__ float s_g[kC], s_b[kC];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int c = blockIdx.x, h = blockIdx.y;
    const int kh = h / a.rep;
    const int t0 = a.t0 + c * kC;
    const int nt = min(kC, a.t0 + a.nt - t0);
    float* ws = a.ws + ((size_t)c * a.Hv + h) * kGdnChunkFloats;
    uint16_t* wW = reinterpret_cast<uint16_t*>(ws);
    uint16_t* wP = reinterpret_cast<uint16_t*>(ws + kC * kD);
    uint16_t* wT = reinterpret_cast<uint16_t*>(ws + kC * kD + kC * kC);
    float* wG = ws + kC * kD + 2 * kC * kC;

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
        s_g[lane] = gv;
        s_b[lane] = bv;
        wG[lane] = expf(gv);
        wG[kC + lane] = expf(__shfl(gv, kC - 1, kWave) - gv);
    }
    // q and k rows of the chunk (zero past the sequence); K also transposed
    for (int i = threadIdx.x; i < kC * (kD / 8); i += blockDim.x) {
        const int t = i / (kD / 8), j = (i - t * (kD / 8)) * 8;
        u32x4 kk = {0u, 0u, 0u, 0u}, qq = {0u, 0u, 0u, 0u};
        if (t < nt) {
            const size_t off = ((size_t)(t0 + t) * a.Hk + kh) * kD + j;
            kk = load_u32x4(a.k + off);
            qq = load_u32x4(a.q + off);
        }
        *reinterpret_cast<u32x4*>(&s_k[t][j]) = kk;
        *reinterpret_cast<u32x4*>(&s_q[t][j]) = qq;
        const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s_kt[j + 2 * e][t] = (uint16_t)(kw[e] & 0xFFFFu);
            s_kt[j + 2 * e + 1][t] = (uint16_t)(kw[e] >> 16);
        }
    }
    __syncthreads();

    // K K^T and Q K^T, rows t of this wavefront's block, blocks s <= t only
    {
        const int tl = lane & 15, ks = (lane >> 4) * 4;
        f32x4 kk[4], qk[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) { kk[sb] = f32x4{0.f, 0.f, 0.f, 0.f}; qk[sb] = kk[sb]; }
#pragma unroll
        for (int j0 = 0; j0 < kD; j0 += 16) {
            const s16x4 ak = load_bf16x4(&s_k[16 * wave + tl][j0 + ks]);
            const s16x4 aq = load_bf16x4(&s_q[16 * wave + tl][j0 + ks]);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb > wave) continue;
                const s16x4 b = load_bf16x4(&s_k[16 * sb + tl][j0 + ks]);
                kk[sb] = mfma16(ak, b, kk[sb]);
                qk[sb] = mfma16(aq, b, qk[sb]);
            }
        }
        // masks and decays: A (strictly lower, times beta_t) to LDS, Pm (lower) to the workspace
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const int s = 16 * sb + tl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * wave + ks + r;
                const float dec = (s <= t) ? expf(s_g[t] - s_g[s]) : 0.f;
                const float av = (sb <= wave && s < t) ? s_b[t] * dec * kk[sb][r] : 0.f;
                const float pv = (sb <= wave) ? dec * qk[sb][r] : 0.f;
                s_a[t][s] = av;
                store_split(wP, kC, t, s, pv);
            }
        }
    }
    __syncthreads();

    // Tinv = (I + A)^-1 by forward substitution: lane c holds column c
    if (wave == 0) {
        // four independent partial sums per row shorten the dependent chain
        float x[kC];
#pragma unroll
        for (int t = 0; t < kC; ++t) {
            float acc0 = (t == lane) ? 1.f : 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll
            for (int s = 0; s < t; s += 4) {
                const float4 av = *reinterpret_cast<const float4*>(&s_a[t][s]);
                acc0 = fmaf(-av.x, x[s], acc0);
                if (s + 1 < t) acc1 = fmaf(-av.y, x[s + 1], acc1);
                if (s + 2 < t) acc2 = fmaf(-av.z, x[s + 2], acc2);
                if (s + 3 < t) acc3 = fmaf(-av.w, x[s + 3], acc3);
            }
            x[t] = (acc0 + acc1) + (acc2 + acc3);
        }
        // Tb = Tinv diag(beta) to the workspace, Tbg = Tinv diag(beta gamma) to LDS
        // (over A, which only this wavefront has been reading)
        const float bc = s_b[lane];
        const float bgc = bc * expf(s_g[lane]);
#pragma unroll
        for (int t = 0; t < kC; ++t) {
            store_split(wT, kC, t, lane, x[t] * bc);
            s_a[t][lane] = x[t] * bgc;
        }
    }
    __syncthreads();

    // W = Tbg K: rows t of this wavefront's block, all 128 key columns
    {
        const int tl = lane & 15, ks = (lane >> 4) * 4;
#pragma unroll
        for (int jb = 0; jb < kD / 16; ++jb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < kC; s0 += 16) {
                const float4 t4 = *reinterpret_cast<const float4*>(&s_a[16 * wave + tl][s0 + ks]);
                const Split4 at = split4(f32x4{t4.x, t4.y, t4.z, t4.w});
                const s16x4 b = load_bf16x4(&s_kt[16 * jb + tl][s0 + ks]);
                acc = mma2(at, b, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) store_split(wW, kD, 16 * wave + ks + r, 16 * jb + tl, acc[r]);
        }
    }
}

// ---------------------------------------------------------------------------
// k_gdn_chunk_scan
// ---------------------------------------------------------------------------
// Operands of one chunk for one wavefront (token rows 16 wave .. + 15), loaded
// one chunk ahead so that their memory latency overlaps the current chunk.
struct ChunkOperands {
    u32x4 w[kD / 16];        // W rows, split pairs (four key columns each)
    u32x4 p[kC / 16];        // Pm rows (blocks above the diagonal unused)
    u32x4 tb[kC / 16];       // Tb rows
    u32x2 q[kD / 16];        // Q rows (bf16)
    u32x2 v;                 // this thread's share of the chunk's V rows (staged to LDS)
    u32x4 k[4];              // this thread's share of the chunk's K (staged to LDS)
    float g;                 // gamma (threads 0..63) or d (threads 64..127) of token threadIdx % 64
};

__device__ __forceinline__ void load_chunk(ChunkOperands& o, const GdnChunkArgs& a, int c, int h, int kh,
                                           int wave, int tl, int ks, int iv) {
    const int t0 = a.t0 + c * kC;
    const int nt = min(kC, a.t0 + a.nt - t0);
    const float* ws = a.ws + ((size_t)c * a.Hv + h) * kGdnChunkFloats;
    const uint16_t* wW = reinterpret_cast<const uint16_t*>(ws);
    const uint16_t* wP = reinterpret_cast<const uint16_t*>(ws + kC * kD);
    const uint16_t* wT = reinterpret_cast<const uint16_t*>(ws + kC * kD + kC * kC);
    const float* wG = ws + kC * kD + 2 * kC * kC;
    const int tw = 16 * wave + tl;
#pragma unroll
    for (int jb = 0; jb < kD / 16; ++jb)
        o.w[jb] = *reinterpret_cast<const u32x4*>(wW + ((size_t)tw * (kD / 4) + (16 * jb + ks) / 4) * 8);
#pragma unroll
    for (int sb = 0; sb < kC / 16; ++sb) {
        const size_t gi = ((size_t)tw * (kC / 4) + (16 * sb + ks) / 4) * 8;
        o.p[sb] = (sb <= wave) ? *reinterpret_cast<const u32x4*>(wP + gi) : u32x4{0u, 0u, 0u, 0u};
        o.tb[sb] = *reinterpret_cast<const u32x4*>(wT + gi);
    }
    const bool qok = tw < nt;
    const uint16_t* qrow = a.q + ((size_t)(t0 + (qok ? tw : 0)) * a.Hk + kh) * kD;
#pragma unroll
    for (int jb = 0; jb < kD / 16; ++jb)
        o.q[jb] = qok ? *reinterpret_cast<const u32x2*>(qrow + 16 * jb + ks) : u32x2{0u, 0u};
    {
        // V of the workgroup's 16 value rows: token threadIdx / 4, rows 4 (threadIdx % 4) .. + 3
        const int t = threadIdx.x >> 2, m = threadIdx.x & 3;
        o.v = (t < nt) ? *reinterpret_cast<const u32x2*>(a.v + ((size_t)(t0 + t) * a.Hv + h) * kD + (iv - tl) + 4 * m)
                       : u32x2{0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = threadIdx.x + u * 256;           // 1024 pieces of 8 bf16: token i / 16, columns 8 (i % 16)
        const int t = i >> 4, j = (i & 15) * 8;
        o.k[u] = (t < nt) ? load_u32x4(a.k + ((size_t)(t0 + t) * a.Hk + kh) * kD + j) : u32x4{0u, 0u, 0u, 0u};
    }
    o.g = (threadIdx.x < 2 * kC) ? wG[threadIdx.x] : 0.f;
}

__global__ __launch_bounds__(256) void k_gdn_chunk_scan(GdnChunkArgs a) {
    __shared__ __attribute__((aligned(16))) u32x4 s_s[kD / 16][kWave];     // S^T blocks, split pairs
    __shared__ __attribute__((aligned(16))) u32x4 s_us[kC / 16][kWave];    // U blocks, split pairs
    __shared__ __attribute__((aligned(16))) u32x4 s_du[kC / 16][kWave];    // d U blocks, split pairs
    __shared__ __attribute__((aligned(16))) uint16_t s_kt[2][kD][kC + 4];  // K transposed, two chunks
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kRB][kC + 4]; // V rows transposed, two chunks
    __shared__ float s_g[2][2 * kC];                                          // gamma, then d
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int h = blockIdx.x % a.Hv;
    const int i0 = (blockIdx.x / a.Hv) * kRB;
    const int kh = h / a.rep;
    const int tl = lane & 15, ks = (lane >> 4) * 4;
    const int iv = i0 + tl;                       // this lane's value row
    float* state = a.state + (size_t)h * kD * kD;
    auto split_pack = [](const f32x4& x) {
        const Split4 sp = split4(x);
        const u32x2 hi = __builtin_bit_cast(u32x2, sp.hi), lo = __builtin_bit_cast(u32x2, sp.lo);
        return u32x4{hi.x, hi.y, lo.x, lo.y};
    };
    auto unpack = [](const u32x4& v) {
        Split4 r;
        r.hi = __builtin_bit_cast(s16x4, u32x2{v.x, v.y});
        r.lo = __builtin_bit_cast(s16x4, u32x2{v.z, v.w});
        return r;
    };
    auto stage = [&](const ChunkOperands& o, int buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = threadIdx.x + u * 256;
            const int t = i >> 4, j = (i & 15) * 8;
            const uint32_t kw[4] = {o.k[u].x, o.k[u].y, o.k[u].z, o.k[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s_kt[buf][j + 2 * e][t] = (uint16_t)(kw[e] & 0xFFFFu);
                s_kt[buf][j + 2 * e + 1][t] = (uint16_t)(kw[e] >> 16);
            }
        }
        {
            const int t = threadIdx.x >> 2, m = threadIdx.x & 3;
            s_vt[buf][4 * m][t] = (uint16_t)(o.v.x & 0xFFFFu);
            s_vt[buf][4 * m + 1][t] = (uint16_t)(o.v.x >> 16);
            s_vt[buf][4 * m + 2][t] = (uint16_t)(o.v.y & 0xFFFFu);
            s_vt[buf][4 * m + 3][t] = (uint16_t)(o.v.y >> 16);
        }
        if (threadIdx.x < 2 * kC) s_g[buf][threadIdx.x] = o.g;
    };

    // S^T blocks jb = 2 wave, 2 wave + 1: lane holds S[iv][16 jb + ks .. + 3]
    f32x4 sm[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int jb = 2 * wave + q;
        const float4 v = *reinterpret_cast<const float4*>(state + (size_t)iv * kD + 16 * jb + ks);
        sm[q] = f32x4{v.x, v.y, v.z, v.w};
        s_s[jb][lane] = split_pack(sm[q]);
    }

    const int nch = (a.nt + kC - 1) / kC;
    ChunkOperands cur, nxt;
    load_chunk(cur, a, 0, h, kh, wave, tl, ks, iv);
    stage(cur, 0);
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        const int t0 = a.t0 + c * kC;
        const int nt = min(kC, a.t0 + a.nt - t0);
        if (c + 1 < nch) load_chunk(nxt, a, c + 1, h, kh, wave, tl, ks, iv);   // in flight during this chunk
        __syncthreads();          // this chunk's K and G are staged; the state blocks are current

        // U = Tb V - W S^T and QS = Q S^T for token rows 16 wave .. + 15, as five
        // independent accumulation chains
        f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = u0, u2 = u0, q0 = u0, q1 = u0;
#pragma unroll
        for (int sb = 0; sb < kC / 16; ++sb)
            u0 = mma2(unpack(cur.tb[sb]), load_bf16x4(&s_vt[buf][tl][16 * sb + ks]), u0);
#pragma unroll
        for (int jb = 0; jb < kD / 16; jb += 2) {
            const Split4 sa = unpack(s_s[jb][lane]), sb = unpack(s_s[jb + 1][lane]);
            u1 = mma3(neg(unpack(cur.w[jb])), sa, u1);
            u2 = mma3(neg(unpack(cur.w[jb + 1])), sb, u2);
            q0 = mma2(__builtin_bit_cast(s16x4, cur.q[jb]), sa, q0);
            q1 = mma2(__builtin_bit_cast(s16x4, cur.q[jb + 1]), sb, q1);
        }
        f32x4 u, qs, du;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            u[r] = u0[r] + (u1[r] + u2[r]);
            qs[r] = q0[r] + q1[r];
            du[r] = u[r] * s_g[buf][kC + 16 * wave + ks + r];
        }
        s_us[wave][lane] = split_pack(u);
        s_du[wave][lane] = split_pack(du);
        __syncthreads();          // every U block written; every state block read

        // O = Gamma QS + Pm U for this wavefront's token rows
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = s_g[buf][16 * wave + ks + r] * qs[r];
#pragma unroll
        for (int sb = 0; sb < kC / 16; ++sb)
            if (sb <= wave) o = mma3(unpack(cur.p[sb]), unpack(s_us[sb][lane]), o);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * wave + ks + r;
            if (t < nt) a.out[((size_t)(t0 + t) * a.Hv + h) * kD + iv] = (uint16_t)f32_to_bf16(o[r]);
        }
        // S^T <- gamma_63 S^T + K^T diag(d) U on key blocks 2 wave, 2 wave + 1
        const float gend = s_g[buf][kC - 1];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int jb = 2 * wave + q;
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gend * sm[q][r];
#pragma unroll
            for (int tb = 0; tb < kC / 16; ++tb)
                acc = mma2(load_bf16x4(&s_kt[buf][16 * jb + tl][16 * tb + ks]), unpack(s_du[tb][lane]), acc);
            sm[q] = acc;
            s_s[jb][lane] = split_pack(acc);   // read after the next chunk's first barrier
        }
        if (c + 1 < nch) {
            stage(nxt, buf ^ 1);               // the other buffer: last read two barriers ago
            cur = nxt;
        }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int jb = 2 * wave + q;
        *reinterpret_cast<float4*>(state + (size_t)iv * kD + 16 * jb + ks) =
            float4{sm[q][0], sm[q][1], sm[q][2], sm[q][3]};
    }
}

size_t gdn_chunked_workspace_floats(int T, int Hv) {
    const int seg = T < kGdnSegT ? T : kGdnSegT;
    return (size_t)((seg + kC - 1) / kC) * (size_t)Hv * kGdnChunkFloats;
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
        tm.launch(k_gdn_chunk_scan, dim3(a.Hv * (kD / kRB)), dim3(256), 0, st, a);
        tm.after();
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace moe_w4
