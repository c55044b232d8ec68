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
//  * large T (prefill): logits tile kernel -> per-token top-k kernel (wavefront
//    per token, atomic histogram and token bitmask) -> per-expert kernel that
//    derives its offset and writes its permutation segment in token order.
#include "device.h"
#include "kernels.h"

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

template <int EPL>
__device__ int wave_topk(float (&vals)[EPL], int E, int k, int lane,
                         int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                         int32_t* ids_lds) {
    int sel_e[kMaxTopK];
    float sel_v[kMaxTopK];
    uint32_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) key[j] = order_key(vals[j]);
    uint32_t taken = 0;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (r >= k) { sel_e[r] = 0x7FFFFFFF; sel_v[r] = 0.f; continue; }
        uint32_t bk = 0u;
        int be = 0x7FFFFFFF;
        float bv = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + kWave * j;
            const bool ok = e < E && !((taken >> j) & 1u);
            if (ok && (be == 0x7FFFFFFF || key[j] > bk || (key[j] == bk && e < be))) {
                bk = key[j]; be = e; bv = vals[j];
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const uint32_t ok_ = __shfl_xor(bk, o, kWave);
            const int oe = __shfl_xor(be, o, kWave);
            const float ov = __shfl_xor(bv, o, kWave);
            if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || ok_ > bk || (ok_ == bk && oe < be))) {
                bk = ok_; be = oe; bv = ov;
            }
        }
        sel_e[r] = be;
        sel_v[r] = bv;
        if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
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

    // phase 1: logits[t][e] for the experts of this wavefront
    for (int e = gw; e < E; e += nw) {
        float acc[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) acc[t] = 0.f;
        const float* wrow = Wr + (size_t)e * H;
        for (int h = lane * 4; h < H; h += kWave * 4) {
            const float4 wv = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                if (t < T) {
                    const u32x2 xv = *reinterpret_cast<const u32x2*>(x + (size_t)t * H + h);
                    acc[t] = fmaf(bf16lo(xv.x), wv.x, acc[t]);
                    acc[t] = fmaf(bf16hi(xv.x), wv.y, acc[t]);
                    acc[t] = fmaf(bf16lo(xv.y), wv.z, acc[t]);
                    acc[t] = fmaf(bf16hi(xv.y), wv.w, acc[t]);
                }
            }
        }
        const float bias = br ? br[e] : 0.f;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {
                const float s = wave_sum(acc[t]);
                if (lane == 0)
                    __hip_atomic_store(&logits[t * E + e], s + bias, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // phase 2: the last workgroup to finish selects and groups
    __shared__ int s_last;
    __shared__ int32_t s_ids[TMAX * kMaxTopK];
    __shared__ int32_t s_cnt[1024];
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    for (int t = wave; t < T; t += kSmallRouteThreads / kWave) {
        float vals[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + kWave * j;
            vals[j] = (e < E) ? __hip_atomic_load(&logits[t * E + e], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : -INFINITY;
        }
        wave_topk<EPL>(vals, E, k, lane, ids + t * k, tw + t * k, s_ids + t * k);
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
constexpr int kLogTileT = 64;
constexpr int kLogTileE = 64;
constexpr int kLogTileK = 32;

// logits[t][e] for a 64x64 tile, fp32 FMA; also clears the histogram and bitmask.
__global__ __launch_bounds__(256) void k_router_logits(
    const uint16_t* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ br,
    int T, int H, int E, float* __restrict__ logits,
    int32_t* __restrict__ counts, uint32_t* __restrict__ bitmask, int bitmask_words) {
    __shared__ float xs[kLogTileT][kLogTileK + 1];
    __shared__ float ws[kLogTileE][kLogTileK + 1];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.y * kLogTileT;
    const int e0 = blockIdx.x * kLogTileE;

    // clearing of the histogram state used by the next kernel
    {
        const int nblk = gridDim.x * gridDim.y;
        const int b = blockIdx.y * gridDim.x + blockIdx.x;
        for (int i = b * 256 + tid; i < bitmask_words; i += nblk * 256) bitmask[i] = 0u;
        for (int i = b * 256 + tid; i < E; i += nblk * 256) counts[i] = 0;
    }

    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4] = {};
    const int lr = tid >> 2, lk = (tid & 3) * 8;
    for (int kb = 0; kb < H; kb += kLogTileK) {
        {   // stage x (bf16 -> fp32) and W_r
            const int t = t0 + lr;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t < T) v = load_u32x4(x + (size_t)t * H + kb + lk);
            xs[lr][lk + 0] = bf16lo(v.x); xs[lr][lk + 1] = bf16hi(v.x);
            xs[lr][lk + 2] = bf16lo(v.y); xs[lr][lk + 3] = bf16hi(v.y);
            xs[lr][lk + 4] = bf16lo(v.z); xs[lr][lk + 5] = bf16hi(v.z);
            xs[lr][lk + 6] = bf16lo(v.w); xs[lr][lk + 7] = bf16hi(v.w);
            const int e = e0 + lr;
            float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            if (e < E) {
                a = *reinterpret_cast<const float4*>(Wr + (size_t)e * H + kb + lk);
                b = *reinterpret_cast<const float4*>(Wr + (size_t)e * H + kb + lk + 4);
            }
            ws[lr][lk + 0] = a.x; ws[lr][lk + 1] = a.y; ws[lr][lk + 2] = a.z; ws[lr][lk + 3] = a.w;
            ws[lr][lk + 4] = b.x; ws[lr][lk + 5] = b.y; ws[lr][lk + 6] = b.z; ws[lr][lk + 7] = b.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kLogTileK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[ty * 4 + i][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[tx * 4 + j][kk];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (br ? br[e] : 0.f);
        }
    }
}

// One wavefront per token: top-k, weights, histogram, token bitmask per expert.
template <int EPL>
__global__ __launch_bounds__(256) void k_router_topk(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ tw, int32_t* __restrict__ counts,
    uint32_t* __restrict__ bitmask, int words_per_expert) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * 4 + (threadIdx.x / kWave);
    if (t >= T) return;
    float vals[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + kWave * j;
        vals[j] = (e < E) ? logits[(size_t)t * E + e] : -INFINITY;
    }
    const int e = wave_topk<EPL>(vals, E, k, lane, ids + (size_t)t * k, tw + (size_t)t * k, nullptr);
    if (lane < k) {
        atomicAdd(&counts[e], 1);
        atomicOr(&bitmask[(size_t)e * words_per_expert + (t >> 5)], 1u << (t & 31));
    }
}

// One workgroup per expert: offset from the histogram, permutation segment in token order.
__global__ __launch_bounds__(256) void k_router_perm(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts,
    const uint32_t* __restrict__ bitmask, int T, int E, int k, int words_per_expert,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
    __shared__ int s_red[256];
    __shared__ int s_scan[256];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    int part = 0;
    for (int i = tid; i < e; i += 256) part += counts[i];
    s_red[tid] = part;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) s_red[tid] += s_red[tid + s];
        __syncthreads();
    }
    const int base = s_red[0];
    if (tid == 0) {
        offsets[e] = base;
        if (e == E - 1) offsets[E] = T * k;
    }
    // contiguous word range per thread, exclusive scan of popcounts
    const int W = words_per_expert;
    const int per = (W + 255) / 256;
    const int w0 = min(tid * per, W), w1 = min(w0 + per, W);
    const uint32_t* row = bitmask + (size_t)e * W;
    int c = 0;
    for (int w = w0; w < w1; ++w) c += __popc(row[w]);
    s_scan[tid] = c;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int v = (tid >= o) ? s_scan[tid - o] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    int pos = base + s_scan[tid] - c;
    for (int w = w0; w < w1; ++w) {
        uint32_t bits = row[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            const int t = w * 32 + b;
            int slot = 0;
            for (int j = 0; j < k; ++j) slot = (ids[(size_t)t * k + j] == e) ? j : slot;
            perm[pos++] = t * k + slot;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int EPL>
static void route_small_epl(const RouteArgs& a, hipStream_t st) {
    if (a.T <= 1)
        hipLaunchKernelGGL((k_route_small<1, EPL>), dim3(kSmallRouteBlocks), dim3(kSmallRouteThreads),
                           0, st, a.x, a.Wr, a.br, a.T, a.H, a.E, a.k, a.ids, a.w, a.counts,
                           a.offsets, a.perm, a.ws_logits, a.ws_ticket);
    else
        hipLaunchKernelGGL((k_route_small<kSmallRouteMaxT, EPL>), dim3(kSmallRouteBlocks),
                           dim3(kSmallRouteThreads), 0, st, a.x, a.Wr, a.br, a.T, a.H, a.E, a.k,
                           a.ids, a.w, a.counts, a.offsets, a.perm, a.ws_logits, a.ws_ticket);
}

hipError_t launch_route_small(const RouteArgs& a, hipStream_t st, KernelTimer& tm) {
    tm.before();
    if (a.E <= 256) route_small_epl<4>(a, st);
    else if (a.E <= 512) route_small_epl<8>(a, st);
    else route_small_epl<16>(a, st);
    tm.after();
    return hipGetLastError();
}

hipError_t launch_route_large(const RouteArgs& a, hipStream_t st, KernelTimer& tm) {
    const int wpe = (a.T + 31) / 32;
    dim3 g1((a.E + kLogTileE - 1) / kLogTileE, (a.T + kLogTileT - 1) / kLogTileT);
    tm.before();
    hipLaunchKernelGGL(k_router_logits, g1, dim3(256), 0, st, a.x, a.Wr, a.br, a.T, a.H, a.E,
                       a.ws_logits, a.counts, a.ws_bitmask, wpe * a.E);
    tm.after();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    if (a.E <= 256)
        hipLaunchKernelGGL(k_router_topk<4>, dim3((a.T + 3) / 4), dim3(256), 0, st, a.ws_logits,
                           a.T, a.E, a.k, a.ids, a.w, a.counts, a.ws_bitmask, wpe);
    else if (a.E <= 512)
        hipLaunchKernelGGL(k_router_topk<8>, dim3((a.T + 3) / 4), dim3(256), 0, st, a.ws_logits,
                           a.T, a.E, a.k, a.ids, a.w, a.counts, a.ws_bitmask, wpe);
    else
        hipLaunchKernelGGL(k_router_topk<16>, dim3((a.T + 3) / 4), dim3(256), 0, st, a.ws_logits,
                           a.T, a.E, a.k, a.ids, a.w, a.counts, a.ws_bitmask, wpe);
    tm.after();
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    hipLaunchKernelGGL(k_router_perm, dim3(a.E), dim3(256), 0, st, a.ids, a.counts, a.ws_bitmask,
                       a.T, a.E, a.k, wpe, a.offsets, a.perm);
    tm.after();
    return hipGetLastError();
}

}  // namespace moe_w4
