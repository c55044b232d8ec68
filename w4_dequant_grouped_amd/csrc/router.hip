// GPU-resident routing for the W4 MoE block (gfx950).
//
// A router picks top_k of E experts for every token ("Perplexity built an
// inference engine for one model, one chip", paragraph 2) and the whole step --
// logits, softmax, top-k, renormalisation, per-expert histogram, offsets and the
// token permutation -- stays on the device with no host round trip (same page,
// paragraph 3: routing is never handed back to the CPU).
//
// Two launch plans:
//  * small T (decode, verification rows): one launch.  Every wavefront of the
//    grid streams a slice of the router weight (reading W_r is a large share of
//    a decode step's bytes, so it is spread over many CUs); the last workgroup to
//    finish (ticket counter in the workspace control block) selects and groups.
//  * large T (prefill): logits on bf16 MFMA from an exact three-way bf16 split
//    of W_r (made inside the logits kernel, or by a kernel of its own for the
//    fallback logits kernel) -> per-token top-k (wavefront per token) ->
//    per-expert kernel that derives its own offset and writes its permutation
//    segment in token order (no atomics, no histogram shared between
//    workgroups).
#include "device.h"
#include "kernels.h"
#include "lds_copy.h"
#include "topk.h"

namespace moe_w4 {

// ---------------------------------------------------------------------------
// small-T router: one launch
// ---------------------------------------------------------------------------
constexpr int kSmallRouteBlocks = 64;   // 256 wavefronts stream W_r
constexpr int kSmallRouteThreads = 256;

template <int TMAX, int EPL>
__global__ __launch_bounds__(kSmallRouteThreads) void k_route_small(
    const uint16_t* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ br,
    int T, int H, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ tw, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    float* __restrict__ logits, uint32_t* __restrict__ ticket) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int gw = blockIdx.x * (kSmallRouteThreads / kWave) + wave;
    const int nw = gridDim.x * (kSmallRouteThreads / kWave);

    // phase 1: logits[t][e] for the experts of this wavefront; all of a lane's
    // W_r and x loads for up to 2048 columns are issued before any is used
    for (int e = gw; e < E; e += nw) {
        float acc[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) acc[t] = 0.f;
        const float* wrow = Wr + (size_t)e * H;
        for (int h0 = 0; h0 < H; h0 += kWave * 4 * 8) {
            float4 wv[8];
            u32x2 xv[8][TMAX];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int h = h0 + (u * kWave + lane) * 4;
                const bool ok = h < H;
                wv[u] = ok ? *reinterpret_cast<const float4*>(wrow + h) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < TMAX; ++t)
                    xv[u][t] = (ok && t < T) ? *reinterpret_cast<const u32x2*>(x + (size_t)t * H + h)
                                             : u32x2{0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int t = 0; t < TMAX; ++t) {
                    acc[t] = fmaf(bf16lo(xv[u][t].x), wv[u].x, acc[t]);
                    acc[t] = fmaf(bf16hi(xv[u][t].x), wv[u].y, acc[t]);
                    acc[t] = fmaf(bf16lo(xv[u][t].y), wv[u].z, acc[t]);
                    acc[t] = fmaf(bf16hi(xv[u][t].y), wv[u].w, acc[t]);
                }
        }
        const float bias = br ? br[e] : 0.f;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {
                const float sum = wave_sum(acc[t]);
                if (lane == 0)
                    __hip_atomic_store(&logits[t * E + e], sum + bias, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // phase 2: the last workgroup to finish selects and groups.  The logits are
    // written and read with device-scope atomics, which bypass the per-XCD
    // caches; each wavefront waits for its own stores to complete before the
    // workgroup takes its ticket, so the workgroup drawing the last ticket sees
    // every logit.  (A full device fence here would also write back the L2.)
    __shared__ int s_last;
    __shared__ int32_t s_ids[TMAX * kMaxTopK];
    __shared__ int32_t s_cnt[1024];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1);
        if (prev >= gridDim.x) {
            // a ticket past the grid: the control block was dirty when this call
            // began; count it and clear the ticket for the next call
            __hip_atomic_fetch_add(ticket + kCtlErrors, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (!s_last) return;

    for (int t = wave; t < T; t += kSmallRouteThreads / kWave) {
        float vals[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + kWave * j;
            vals[j] = (e < E) ? __hip_atomic_load(&logits[t * E + e], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : -INFINITY;
        }
        wave_topk_select<EPL>(vals, E, k, lane, ids + t * k, tw + t * k, s_ids + t * k);
    }
    // grouping of the T*k (token, slot) entries
    for (int i = threadIdx.x; i < E; i += blockDim.x) s_cnt[i] = 0;
    __syncthreads();
    const int n = T * k;
    for (int i = threadIdx.x; i < n; i += blockDim.x) atomicAdd(&s_cnt[s_ids[i]], 1);
    __syncthreads();
    // exclusive scan of the E counters by one wavefront (E <= 1024: 16 per lane)
    if (wave == 0) {
        int local[16];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane * 16 + j;
            local[j] = (e < E) ? s_cnt[e] : 0;
            sum += local[j];
        }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int v = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += v;
        }
        int run = incl - sum;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane * 16 + j;
            if (e < E) {
                counts[e] = local[j];
                offsets[e] = run;
                s_cnt[e] = run;        // s_cnt now holds segment starts
            }
            run += local[j];
        }
        if (lane == kWave - 1) offsets[E] = run;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int e = s_ids[i];
        const int t = i / k;
        int rank = 0;
        for (int tp = 0; tp < t; ++tp)
            for (int j = 0; j < k; ++j) rank += (s_ids[tp * k + j] == e) ? 1 : 0;
        perm[s_cnt[e] + rank] = i;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// large-T router
// ---------------------------------------------------------------------------
// x is bf16, so x . w for fp32 w equals x . hi + x . mid + x . lo exactly when
// w = hi + mid + lo with hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid)
// (24 significand bits = 3 x 8; each product of two bf16 is exact in fp32).  The
// logits then run on bf16 MFMA with fp32 accumulation.

// W_r [E][H] fp32 -> three bf16 planes [3][E][H].
__global__ __launch_bounds__(256) void k_router_split(const float* __restrict__ Wr, long n,
                                                      uint16_t* __restrict__ planes) {
    for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (long)gridDim.x * 256 * 4) {
        const float4 w = *reinterpret_cast<const float4*>(Wr + i);
        const float v[4] = {w.x, w.y, w.z, w.w};
        uint32_t hi[2], mid[2], lo[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float h0 = bf16_to_f32(f32_to_bf16(v[2 * q])), h1 = bf16_to_f32(f32_to_bf16(v[2 * q + 1]));
            float r0 = v[2 * q] - h0, r1 = v[2 * q + 1] - h1;
            float m0 = bf16_to_f32(f32_to_bf16(r0)), m1 = bf16_to_f32(f32_to_bf16(r1));
            hi[q] = pack_bf16x2(h0, h1);
            mid[q] = pack_bf16x2(m0, m1);
            lo[q] = pack_bf16x2(r0 - m0, r1 - m1);
        }
        *reinterpret_cast<u32x2*>(planes + i) = u32x2{hi[0], hi[1]};
        *reinterpret_cast<u32x2*>(planes + n + i) = u32x2{mid[0], mid[1]};
        *reinterpret_cast<u32x2*>(planes + 2 * n + i) = u32x2{lo[0], lo[1]};
    }
}

// Partial logits over one eighth of H (kRouterKSplit) for a tile of 256 tokens x
// 64 experts: wavefront w owns tokens 64w..64w+63 (four 16-token MFMA row blocks)
// and all 64 experts (four 16-expert blocks, three planes each), so every step's
// 16 operand loads feed 48 MFMAs.  MFMA 16x16x32 bf16 operands come straight from
// global memory (the four wavefronts share the weight fragments through L1):
// lane l holds row (token or expert) l%16 and the 8 consecutive k at 8*(l/16)
// of each 32-k step.  The next step's operands are loaded while the current
// step's MFMAs run.  The top-k kernel adds the partials in a fixed order.
constexpr int kLgTokW = 64;                  // tokens per wavefront
constexpr int kLgTok = 4 * kLgTokW;          // tokens per workgroup
constexpr int kLgExp = 64;                   // experts per workgroup

struct LgFrag {
    bf16x8 a[4];
    bf16x8 b[4][3];
};

__device__ __forceinline__ void lg_load(LgFrag& f, const uint16_t* const (&xa)[4],
                                        const uint16_t* const (&wb)[4], size_t plane, int k) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) f.a[mb] = *reinterpret_cast<const bf16x8*>(xa[mb] + k);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int p = 0; p < 3; ++p)
            f.b[nb][p] = *reinterpret_cast<const bf16x8*>(wb[nb] + p * plane + k);
}

__global__ __launch_bounds__(256) void k_router_logits_mfma(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes, int T, int H, int E,
    float* __restrict__ partial) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int t0 = blockIdx.y * kLgTok + wave * kLgTokW;
    if (t0 >= T) return;                       // whole wavefront past T (no barriers below)
    const int e0 = blockIdx.x * kLgExp;
    const int ks = H / kRouterKSplit;          // a multiple of 32 (H % 256 == 0)
    const int kbeg = blockIdx.z * ks;
    const size_t plane = (size_t)E * H;
    const uint16_t* xa[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int trow = min(t0 + mb * 16 + (lane & 15), T - 1);     // rows past T re-read row T-1
        xa[mb] = x + (size_t)trow * H + kbeg + (lane >> 4) * 8;
    }
    const uint16_t* wb[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
        wb[nb] = planes + (size_t)min(e0 + nb * 16 + (lane & 15), E - 1) * H + kbeg + (lane >> 4) * 8;
    f32x4 acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    LgFrag cur;
    lg_load(cur, xa, wb, plane, 0);
    for (int kc = 0; kc < ks; kc += 32) {
        LgFrag nxt;
        if (kc + 32 < ks) lg_load(nxt, xa, wb, plane, kc + 32);
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[mb], cur.b[nb][p],
                                                                         acc[mb][nb], 0, 0, 0);
        cur = nxt;
    }
    float* out = partial + (size_t)blockIdx.z * T * E;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int e = e0 + nb * 16 + (lane & 15);
            if (e >= E) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = t0 + mb * 16 + (lane >> 4) * 4 + q;
                if (t < T) out[(size_t)t * E + e] = acc[mb][nb][q];
            }
        }
}

// Partial logits over one eighth of H for a tile of 128 tokens x 64 experts, with
// both operands staged in LDS (used when H/8 is a multiple of 64).  Each 64-k
// chunk of the 128 activation rows is copied global -> LDS by global_load_lds
// (eight rows of 128 contiguous bytes per instruction, so each instruction reads
// whole cache lines of eight rows); the chunk's 64 x 64 fp32 router weights are
// loaded by the threads (64 contiguous bytes each) and split in registers into
// the three bf16 planes hi + mid + lo, which they write to LDS -- the same split
// as k_router_split, done per workgroup instead of by a kernel of its own.  Two
// stages: while chunk c is multiplied, chunk c+1's rows are copied and its
// weights loaded, and the weights are split into the other stage after the
// MFMAs.  Wavefront (i, j) computes tokens 64i..64i+63 x experts 32j..32j+31
// (four by two 16x16 blocks, three planes each): per 32-k step, 10 LDS operand
// reads feed 24 MFMAs.  A row r of a stage holds its 8 pieces of 16 bytes with
// logical piece p at p ^ ((r>>1)&7), so the 16 rows of an operand read hit 16
// distinct 4-bank groups.
constexpr int kRlTok = 128;                  // tokens per workgroup
constexpr int kRlExp = 64;                   // experts per workgroup
constexpr int kRlKC = 64;                    // k per chunk
constexpr int kRlRow = kRlKC * 2;            // bytes of a row per chunk (128)
constexpr int kRlARows = kRlTok;             // activation rows per stage
constexpr int kRlBRows = 3 * kRlExp;         // weight-plane rows per stage
constexpr int kRlStage = (kRlARows + kRlBRows) * kRlRow;    // 40 KiB
constexpr int kRlRowsPerCopy = 64 * 16 / kRlRow;            // 8 rows per copy instruction
constexpr int kRlACopies = kRlARows / kRlRowsPerCopy / 4;   // per wavefront (4)

__device__ __forceinline__ int rl_swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(256, 2) void k_router_logits_lds(
    const uint16_t* __restrict__ x, const float* __restrict__ Wr, int T, int H, int E,
    float* __restrict__ partial) {
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[2 * kRlStage];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)uniform32(threadIdx.x / kWave);
    const int wi = wave >> 1, wj = wave & 1;
    const int tbase = blockIdx.y * kRlTok;
    const int e0 = blockIdx.x * kRlExp;
    const int ks = H / kRouterKSplit;          // a multiple of kRlKC here
    const int kbeg = blockIdx.z * ks;
    const uint32_t ring = lds_addr(s_stage);

    // activation copies: lane L fills position L&7 of stage row 8q + (L>>3) of copy
    // q with its logical piece; rows past T re-read the last valid row
    const uint64_t xbase = uniform64((uint64_t)(x + kbeg));
    uint32_t a_off[kRlACopies];
#pragma unroll
    for (int i = 0; i < kRlACopies; ++i) {
        const int row = (wave * kRlACopies + i) * kRlRowsPerCopy + (lane >> 3);
        const int logical = (lane & 7) ^ rl_swz(row);
        a_off[i] = (uint32_t)min(tbase + row, T - 1) * (uint32_t)(H * 2) + (uint32_t)logical * 16u;
    }
    auto issue_a = [&](int c, int st) {
        const uint32_t sa = ring + st * kRlStage;
        const uint64_t xa = xbase + (uint64_t)c * kRlRow;
#pragma unroll
        for (int i = 0; i < kRlACopies; ++i)
            dma16_to_lds(xa, a_off[i], sa + (wave * kRlACopies + i) * kRlRowsPerCopy * kRlRow);
    };
    // weights: thread t owns expert row wr = t/4 (past E: the last expert) and k
    // 16 wq .. 16 wq + 15 of each chunk, i.e. logical pieces 2 wq and 2 wq + 1 of
    // that row in each plane
    const int wr = threadIdx.x >> 2, wq = threadIdx.x & 3;
    const float* wsrc = Wr + (size_t)min(e0 + wr, E - 1) * H + kbeg + 16 * wq;
    auto load_w = [&](int c, float4 (&w)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = *reinterpret_cast<const float4*>(wsrc + c * kRlKC + 4 * q);
    };
    auto store_w = [&](const float4 (&w)[4], int st) {
        const float v[16] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w,
                             w[2].x, w[2].y, w[2].z, w[2].w, w[3].x, w[3].y, w[3].z, w[3].w};
        uint32_t hi[8], mid[8], lo[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // w = hi + mid + lo exactly (see k_router_split)
            hi[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
            const float r0 = v[2 * q] - bf16lo(hi[q]), r1 = v[2 * q + 1] - bf16hi(hi[q]);
            mid[q] = pack_bf16x2(r0, r1);
            lo[q] = pack_bf16x2(r0 - bf16lo(mid[q]), r1 - bf16hi(mid[q]));
        }
        uint8_t* sb = s_stage + st * kRlStage + kRlARows * kRlRow;
        const int sw = rl_swz(wr);               // the same for the row in every plane
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int piece = ((2 * wq + h) ^ sw) * 16;
            *reinterpret_cast<u32x4*>(sb + (0 * kRlExp + wr) * kRlRow + piece) =
                u32x4{hi[4 * h], hi[4 * h + 1], hi[4 * h + 2], hi[4 * h + 3]};
            *reinterpret_cast<u32x4*>(sb + (1 * kRlExp + wr) * kRlRow + piece) =
                u32x4{mid[4 * h], mid[4 * h + 1], mid[4 * h + 2], mid[4 * h + 3]};
            *reinterpret_cast<u32x4*>(sb + (2 * kRlExp + wr) * kRlRow + piece) =
                u32x4{lo[4 * h], lo[4 * h + 1], lo[4 * h + 2], lo[4 * h + 3]};
        }
    };

    f32x4 acc[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int r16 = lane & 15, g = lane >> 4;
    const int nch = ks / kRlKC;
    float4 w[4];
    issue_a(0, 0);
    load_w(0, w);
    store_w(w, 0);
    for (int c = 0; c < nch; ++c) {
        const int st = c & 1;
        wait_vmcnt<0>();
        __syncthreads();       // chunk c visible to all; the other stage is free
        const bool more = c + 1 < nch;
        if (more) {
            issue_a(c + 1, st ^ 1);
            load_w(c + 1, w);
        }
        const uint8_t* sa = s_stage + st * kRlStage;
        const uint8_t* sb = sa + kRlARows * kRlRow;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = ((4 * j + g) ^ rl_swz(r16)) * 16;
            bf16x8 a[4], b[2][3];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                a[mb] = *reinterpret_cast<const bf16x8*>(sa + (64 * wi + 16 * mb + r16) * kRlRow + col);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    b[nb][p] = *reinterpret_cast<const bf16x8*>(
                        sb + (p * kRlExp + 32 * wj + 16 * nb + r16) * kRlRow + col);
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b[nb][p], acc[mb][nb],
                                                                             0, 0, 0);
        }
        if (more) store_w(w, st ^ 1);   // the stage read in iteration c-1, free since the barrier
    }
    float* out = partial + (size_t)blockIdx.z * T * E;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int e = e0 + 32 * wj + 16 * nb + r16;
            if (e >= E) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = tbase + 64 * wi + 16 * mb + g * 4 + q;
                if (t < T) out[(size_t)t * E + e] = acc[mb][nb][q];
            }
        }
}

// One wavefront per token: logits = bias + the K-split partials (fixed order),
// then top-k and renormalised weights (no shared state).
template <int EPL>
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ partial,
                                                     const float* __restrict__ br, int T, int E,
                                                     int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ tw, uint8_t* __restrict__ ids8) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * 4 + (threadIdx.x / kWave);
    if (t >= T) return;
    float vals[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + kWave * j;
        float v = -INFINITY;
        if (e < E) {
            static_assert(kRouterKSplit == 8, "summation order below");
            float p[kRouterKSplit];
#pragma unroll
            for (int q = 0; q < kRouterKSplit; ++q) p[q] = partial[((size_t)q * T + t) * E + e];
            v = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            if (br) v += br[e];
        }
        vals[j] = v;
    }
    wave_topk_select<EPL>(vals, E, k, lane, ids + (size_t)t * k, tw + (size_t)t * k, nullptr, nullptr,
                          nullptr, ids8 ? ids8 + (size_t)t * k : nullptr);
}

// One workgroup per expert e.  Every token's ids are ascending, so
//   offsets[e] = sum over tokens of #{j : ids[t][j] < e}
// and the expert's segment lists, in token order, the tokens whose ids contain
// e.  Each workgroup reads all ids (T*k ints, L2-resident) and needs nothing
// from the others: no histogram, no atomics.  Thread tid owns a contiguous run
// of the flattened (t, j) entries, read kGroupBatch x 4 at a time with every
// load of a batch issued together, once to count and, if the run spans more
// than one batch, once more from L2 to write its part of the permutation (a
// run of one batch, T * k <= 65536, stays in registers between the passes).
// 1024 threads keep each thread's run short (at T = 16384 two batches per pass
// instead of eight), since the kernel is bound by its dependent batches of loads.
constexpr int kGroupThreads = 1024;
constexpr int kGroupBatch = 16;          // int4 loads per thread issued together

__device__ __forceinline__ void group_load(const int32_t* __restrict__ ids, int n, int q,
                                           int4& w) {
    const int i = 4 * q;
    if (i + 3 < n) {
        w = *reinterpret_cast<const int4*>(ids + i);
    } else {
        w.x = (i < n) ? ids[i] : 0x7FFFFFFF;
        w.y = (i + 1 < n) ? ids[i + 1] : 0x7FFFFFFF;
        w.z = (i + 2 < n) ? ids[i + 2] : 0x7FFFFFFF;
        w.w = (i + 3 < n) ? ids[i + 3] : 0x7FFFFFFF;
    }
}

__global__ __launch_bounds__(kGroupThreads) void k_router_group(const int32_t* __restrict__ ids,
                                                                int T, int E, int k,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ perm) {
    __shared__ int s_below[kGroupThreads / kWave];
    __shared__ int s_hits[kGroupThreads / kWave];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = T * k;
    const int n4 = (n + 3) / 4;
    const int per4 = (n4 + kGroupThreads - 1) / kGroupThreads;
    const int q0 = min(tid * per4, n4), q1 = min(q0 + per4, n4);
    int below = 0, hits = 0;
    int4 w[kGroupBatch];                 // the last batch read; the whole run when it fits one
    for (int qb = q0; qb < q1; qb += kGroupBatch) {
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            w[u] = int4{0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF};
            if (qb + u < q1) group_load(ids, n, qb + u, w[u]);
        }
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            const bool ok = qb + u < q1;
            below += ok ? (w[u].x < e) + (w[u].y < e) + (w[u].z < e) + (w[u].w < e) : 0;
            hits += ok ? (w[u].x == e) + (w[u].y == e) + (w[u].z == e) + (w[u].w == e) : 0;
        }
    }
    // inclusive scan of hits and sum of below: within the wavefront by shuffles,
    // then across the kGroupThreads / 64 wavefronts
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    int incl = hits, bsum = below;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int vh = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += vh;
        bsum += __shfl_xor(bsum, o, kWave);
    }
    if (lane == kWave - 1) s_hits[wave] = incl;
    if (lane == 0) s_below[wave] = bsum;
    __syncthreads();
    int hits_before = 0, base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kGroupThreads / kWave; ++w) {
        hits_before += (w < wave) ? s_hits[w] : 0;
        total += s_hits[w];
        base += s_below[w];
    }
    int pos = base + hits_before + incl - hits;
    if (tid == 0) {
        offsets[e] = base;
        counts[e] = total;
        if (e == E - 1) offsets[E] = n;
    }
    if (hits == 0) return;
    const bool one_batch = q1 - q0 <= kGroupBatch;
    for (int qb = q0; qb < q1; qb += kGroupBatch) {
        if (!one_batch) {
#pragma unroll
            for (int u = 0; u < kGroupBatch; ++u) {
                w[u] = int4{0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF};
                if (qb + u < q1) group_load(ids, n, qb + u, w[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            if (qb + u >= q1) continue;
            const int i = 4 * (qb + u);
            if (w[u].x == e) perm[pos++] = i;
            if (w[u].y == e) perm[pos++] = i + 1;
            if (w[u].z == e) perm[pos++] = i + 2;
            if (w[u].w == e) perm[pos++] = i + 3;
        }
    }
}

// The same grouping over the ids as bytes (E <= 256), which the top-k kernel
// writes beside the int32 ids: one 16-byte load brings 16 entries instead of 4,
// so a thread's run is a quarter of the bytes and, up to T * k = 131072 (T =
// 16384 at top-8), one batch that stays in registers for the writing pass.
// Entries past T * k in the last 16-byte piece are not counted (every byte
// value is a valid id, so they are masked by position).
constexpr int kGroup8Batch = 8;          // 16-byte loads per thread issued together

__device__ __forceinline__ void count_bytes(uint32_t w, int e, int nvalid, int& below, int& hits) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int v = (int)((w >> (8 * b)) & 0xFFu);
        const bool ok = b < nvalid;
        below += (ok && v < e) ? 1 : 0;
        hits += (ok && v == e) ? 1 : 0;
    }
}

__global__ __launch_bounds__(kGroupThreads) void k_router_group8(const uint8_t* __restrict__ ids8,
                                                                 int T, int E, int k,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ perm) {
    __shared__ int s_below[kGroupThreads / kWave];
    __shared__ int s_hits[kGroupThreads / kWave];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = T * k;
    const int n16 = (n + 15) / 16;
    const int per = (n16 + kGroupThreads - 1) / kGroupThreads;
    const int q0 = min(tid * per, n16), q1 = min(q0 + per, n16);
    int below = 0, hits = 0;
    u32x4 w[kGroup8Batch];               // the last batch read; the whole run when it fits one
    for (int qb = q0; qb < q1; qb += kGroup8Batch) {
#pragma unroll
        for (int u = 0; u < kGroup8Batch; ++u)
            if (qb + u < q1) w[u] = *reinterpret_cast<const u32x4*>(ids8 + 16 * (size_t)(qb + u));
#pragma unroll
        for (int u = 0; u < kGroup8Batch; ++u) {
            if (qb + u >= q1) continue;
            const int nv = n - 16 * (qb + u);          // >= 1 valid entries in this piece
            count_bytes(w[u].x, e, nv, below, hits);
            count_bytes(w[u].y, e, nv - 4, below, hits);
            count_bytes(w[u].z, e, nv - 8, below, hits);
            count_bytes(w[u].w, e, nv - 12, below, hits);
        }
    }
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    int incl = hits, bsum = below;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int vh = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += vh;
        bsum += __shfl_xor(bsum, o, kWave);
    }
    if (lane == kWave - 1) s_hits[wave] = incl;
    if (lane == 0) s_below[wave] = bsum;
    __syncthreads();
    int hits_before = 0, base = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kGroupThreads / kWave; ++v) {
        hits_before += (v < wave) ? s_hits[v] : 0;
        total += s_hits[v];
        base += s_below[v];
    }
    int pos = base + hits_before + incl - hits;
    if (tid == 0) {
        offsets[e] = base;
        counts[e] = total;
        if (e == E - 1) offsets[E] = n;
    }
    if (hits == 0) return;
    const bool one_batch = q1 - q0 <= kGroup8Batch;
    for (int qb = q0; qb < q1; qb += kGroup8Batch) {
        if (!one_batch) {
#pragma unroll
            for (int u = 0; u < kGroup8Batch; ++u)
                if (qb + u < q1) w[u] = *reinterpret_cast<const u32x4*>(ids8 + 16 * (size_t)(qb + u));
        }
#pragma unroll
        for (int u = 0; u < kGroup8Batch; ++u) {
            if (qb + u >= q1) continue;
            const int i0 = 16 * (qb + u);
            const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                const int v = (int)((ww[b >> 2] >> (8 * (b & 3))) & 0xFFu);
                if (i0 + b < n && v == e) perm[pos++] = i0 + b;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int EPL>
static void route_small_epl(const RouteArgs& a, hipStream_t st, KernelTimer& tm) {
    if (a.T <= 1)
        tm.launch((k_route_small<1, EPL>), dim3(kSmallRouteBlocks), dim3(kSmallRouteThreads),
                           0, st, a.x, a.Wr, a.br, a.T, a.H, a.E, a.k, a.ids, a.w, a.counts,
                           a.offsets, a.perm, a.ws_logits, a.ws_ticket);
    else
        tm.launch((k_route_small<kSmallRouteMaxT, EPL>), dim3(kSmallRouteBlocks),
                           dim3(kSmallRouteThreads), 0, st, a.x, a.Wr, a.br, a.T, a.H, a.E, a.k,
                           a.ids, a.w, a.counts, a.offsets, a.perm, a.ws_logits, a.ws_ticket);
}

hipError_t launch_route_small(const RouteArgs& a, hipStream_t st, KernelTimer& tm) {
    tm.before();
    if (a.E <= 256) route_small_epl<4>(a, st, tm);
    else if (a.E <= 512) route_small_epl<8>(a, st, tm);
    else route_small_epl<16>(a, st, tm);
    tm.after();
    return hipGetLastError();
}

hipError_t launch_route_large(const RouteArgs& a, hipStream_t st, KernelTimer& tm) {
    hipError_t err;
    if ((a.H / kRouterKSplit) % kRlKC == 0) {
        // three launches: the logits kernel splits W_r itself
        tm.before();
        tm.launch(k_router_logits_lds,
                  dim3((a.E + kRlExp - 1) / kRlExp, (a.T + kRlTok - 1) / kRlTok, kRouterKSplit),
                  dim3(256), 0, st, a.x, a.Wr, a.T, a.H, a.E, a.ws_logits);
        tm.after();
    } else {
        // four launches: the weight planes first, for the fallback logits kernel
        const long n = (long)a.E * a.H;
        tm.before();
        tm.launch(k_router_split, dim3((unsigned)min((n / 4 + 255) / 256, 1024L)), dim3(256), 0, st,
                  a.Wr, n, a.ws_planes);
        tm.after();
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        tm.before();
        tm.launch(k_router_logits_mfma,
                  dim3((a.E + kLgExp - 1) / kLgExp, (a.T + kLgTok - 1) / kLgTok, kRouterKSplit),
                  dim3(256), 0, st, a.x, a.ws_planes, a.T, a.H, a.E, a.ws_logits);
        tm.after();
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    if (a.E <= 256)
        tm.launch(k_router_topk<4>, dim3((a.T + 3) / 4), dim3(256), 0, st, a.ws_logits, a.br,
                           a.T, a.E, a.k, a.ids, a.w, a.ws_ids8);
    else if (a.E <= 512)
        tm.launch(k_router_topk<8>, dim3((a.T + 3) / 4), dim3(256), 0, st, a.ws_logits, a.br,
                           a.T, a.E, a.k, a.ids, a.w, (uint8_t*)nullptr);
    else
        tm.launch(k_router_topk<16>, dim3((a.T + 3) / 4), dim3(256), 0, st, a.ws_logits, a.br,
                           a.T, a.E, a.k, a.ids, a.w, (uint8_t*)nullptr);
    tm.after();
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    if (a.E <= 256)
        tm.launch(k_router_group8, dim3(a.E), dim3(kGroupThreads), 0, st, (const uint8_t*)a.ws_ids8,
                  a.T, a.E, a.k, a.counts, a.offsets, a.perm);
    else
        tm.launch(k_router_group, dim3(a.E), dim3(kGroupThreads), 0, st, (const int32_t*)a.ids, a.T,
                  a.E, a.k, a.counts, a.offsets, a.perm);
    tm.after();
    return hipGetLastError();
}

}  // namespace moe_w4
