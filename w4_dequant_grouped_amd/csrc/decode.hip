// Decode path of the W4 MoE block (T <= 8 rows), gfx950.
//
// Decode reuses almost no weights across tokens, so it is bound by the bytes it
// reads: the point is to stream each selected expert's packed bytes exactly once
// ("Perplexity's Lily brings fast local AI to Apple silicon Macs", section "Where
// the Engine Gains Speed": decode worked to minimise the bytes moved per token;
// "Perplexity built an inference engine for one model, one chip", paragraph 4:
// verification batches of two to five rows routed to different experts raise the
// weight reads).  Rows that picked the same expert share one read of it.
//
// Each wavefront owns whole weight rows.  A lane holds 32 consecutive codes (one
// 128-bit load) and dots them against the token rows with the per-group affine
// form  sum_k (c s + b) x_k = s * sum_k (128 + c) x_k + (b - 128 s) * sum_k x_k,
// where bf16(128 + c) has the bit pattern 0x4300 | c, so the codes become bf16
// operands of v_dot2_f32_bf16 with two bit operations per pair and no
// conversion; the expanded weights never exist.
//
//   k_decode_gateup: (slot, 16 rows of I) per workgroup -> h = silu(g) * u (bf16)
//   k_decode_down:   8 output rows per workgroup, every slot -> out (bf16)
// A slot is an expert with a non-empty segment (ascending id), then the shared
// expert.  Both kernels read the routing from the device; the grid depends only
// on T.
#include "device.h"
#include "kernels.h"

namespace moe_w4 {

constexpr int kMaxSlots = kDecodeMaxT * 16 + 1;

struct Slot {
    int e;      // expert id, or -1 for the shared expert
    int off;    // first h row of the slot
    int cnt;    // rows (tokens) in the slot
};

// Wavefront 0 lists the non-empty experts (ascending) and then the shared expert.
__device__ __forceinline__ void build_slots(const int32_t* __restrict__ offsets, int E, int T, int k,
                                            int has_shared, Slot* s_slots, int* s_n, int lane) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        int a = 0, b = 0;
        if (e < E) { a = offsets[e]; b = offsets[e + 1]; }
        // a segment is clipped to the T*k routed rows, so malformed offsets cannot
        // send a row index out of range
        const int lim = T * k;
        a = min(max(a, 0), lim);
        b = min(max(b, a), lim);
        const bool active = b > a;
        const uint64_t mask = __ballot(active);
        const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
        if (active && pos < kMaxSlots - 1) s_slots[pos] = Slot{e, a, min(b - a, T)};
        base += __popcll(mask);
    }
    base = min(base, kMaxSlots - 1);
    if (lane == 0) {
        if (has_shared) s_slots[base] = Slot{-1, T * k, T};
        *s_n = base + (has_shared ? 1 : 0);
    }
}

// 32 bf16 of a row (64 bytes at p) -> 16 dwords paired as (x[j], x[j+4]) per 8,
// plus their sum.
__device__ __forceinline__ void load_interleaved32(const uint16_t* p, uint32_t (&xi)[16], float& sum) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const u32x4 v = q[b];   // x[8b .. 8b+7] as 4 natural pairs
        xi[4 * b + 0] = interleave_pair(v.x, v.z, 0);
        xi[4 * b + 1] = interleave_pair(v.x, v.z, 1);
        xi[4 * b + 2] = interleave_pair(v.y, v.w, 0);
        xi[4 * b + 3] = interleave_pair(v.y, v.w, 1);
        s = dot2_bf16(v.x, 0x3F803F80u, s);
        s = dot2_bf16(v.y, 0x3F803F80u, s);
        s = dot2_bf16(v.z, 0x3F803F80u, s);
        s = dot2_bf16(v.w, 0x3F803F80u, s);
    }
    sum = s;
}

// sum_k (128 + c_k) x_k over 32 codes (4 dwords) and the matching interleaved x.
__device__ __forceinline__ float dot32_magic(const u32x4& c, const uint32_t (&xi)[16]) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a0 = dot2_bf16(magic_pair(c.x, j), xi[j], a0);
        a1 = dot2_bf16(magic_pair(c.y, j), xi[4 + j], a1);
        a0 = dot2_bf16(magic_pair(c.z, j), xi[8 + j], a0);
        a1 = dot2_bf16(magic_pair(c.w, j), xi[12 + j], a1);
    }
    return a0 + a1;
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU
// ---------------------------------------------------------------------------
constexpr int kGuRowsPerWave = 4;
constexpr int kGuRowsPerBlock = 4 * kGuRowsPerWave;

template <int TMAX>
__global__ __launch_bounds__(256) void k_decode_gateup(
    const uint16_t* __restrict__ x, int T, int H, int I, int E, int k,
    W4Set routed, W4Set shared, int has_shared,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    uint16_t* __restrict__ h) {
    __shared__ Slot s_slots[kMaxSlots];
    __shared__ int s_n;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (wave == 0) build_slots(offsets, E, T, k, has_shared, s_slots, &s_n, lane);
    __syncthreads();
    if ((int)blockIdx.x >= s_n) return;
    const Slot sl = s_slots[blockIdx.x];
    const bool is_shared = sl.e < 0;
    const int e = is_shared ? 0 : sl.e;
    const W4 G = is_shared ? shared.gate : routed.gate;
    const W4 U = is_shared ? shared.up : routed.up;

    // token of each row of the slot
    int tok[TMAX];
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
        tok[i] = 0;
        if (i < sl.cnt) tok[i] = is_shared ? i : min(max(perm[sl.off + i], 0), T * k - 1) / k;
    }

    const int n0 = blockIdx.y * kGuRowsPerBlock + wave * kGuRowsPerWave;
    const int ngroups = H / kGroup;
    const int nchunks = H / 32;
    float ag[kGuRowsPerWave][TMAX], au[kGuRowsPerWave][TMAX];
#pragma unroll
    for (int r = 0; r < kGuRowsPerWave; ++r)
#pragma unroll
        for (int i = 0; i < TMAX; ++i) { ag[r][i] = 0.f; au[r][i] = 0.f; }

    for (int c = lane; c < nchunks; c += kWave) {
        u32x4 cg[kGuRowsPerWave], cu[kGuRowsPerWave];
        float sg[kGuRowsPerWave], bg[kGuRowsPerWave], su[kGuRowsPerWave], bu[kGuRowsPerWave];
#pragma unroll
        for (int r = 0; r < kGuRowsPerWave; ++r) {
            const size_t row = (size_t)e * I + (n0 + r);
            cg[r] = load_u32x4(G.codes + row * (H / 2) + c * 16);
            cu[r] = load_u32x4(U.codes + row * (H / 2) + c * 16);
            const size_t gi = row * ngroups + (c >> 1);
            sg[r] = bf16_to_f32(G.scales[gi]);
            bg[r] = bf16_to_f32(G.biases[gi]);
            su[r] = bf16_to_f32(U.scales[gi]);
            bu[r] = bf16_to_f32(U.biases[gi]);
        }
#pragma unroll
        for (int i = 0; i < TMAX; ++i) {
            if (i >= sl.cnt) break;
            uint32_t xi[16];
            float xs;
            load_interleaved32(x + (size_t)tok[i] * H + c * 32, xi, xs);
#pragma unroll
            for (int r = 0; r < kGuRowsPerWave; ++r) {
                const float pg = dot32_magic(cg[r], xi);
                const float pu = dot32_magic(cu[r], xi);
                ag[r][i] += fmaf(sg[r], pg, (bg[r] - 128.0f * sg[r]) * xs);
                au[r][i] += fmaf(su[r], pu, (bu[r] - 128.0f * su[r]) * xs);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
        if (i >= sl.cnt) break;
        const int hrow = sl.off + i;
#pragma unroll
        for (int r = 0; r < kGuRowsPerWave; ++r) {
            const float g = wave_sum(ag[r][i]);
            const float u = wave_sum(au[r][i]);
            if (lane == r) h[(size_t)hrow * I + n0 + r] = (uint16_t)f32_to_bf16(silu(g) * u);
        }
    }
}

// ---------------------------------------------------------------------------
// down + weighted combine
// ---------------------------------------------------------------------------
constexpr int kDnRowsPerWave = 2;
constexpr int kDnRowsPerBlock = 4 * kDnRowsPerWave;

template <int TMAX>
__global__ __launch_bounds__(256) void k_decode_down(
    int T, int H, int I, int E, int k, W4Set routed, W4Set shared, int has_shared,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const uint16_t* __restrict__ h,
    uint16_t* __restrict__ out) {
    __shared__ Slot s_slots[kMaxSlots];
    __shared__ int s_n;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (wave == 0) build_slots(offsets, E, T, k, has_shared, s_slots, &s_n, lane);
    __syncthreads();
    const int nslots = s_n;
    const int n0 = blockIdx.x * kDnRowsPerBlock + wave * kDnRowsPerWave;
    const int cpr = I / 32;            // 32-code chunks per down row
    const int ngroups = I / kGroup;

    float acc[kDnRowsPerWave][TMAX];
#pragma unroll
    for (int r = 0; r < kDnRowsPerWave; ++r)
#pragma unroll
        for (int t = 0; t < TMAX; ++t) acc[r][t] = 0.f;

    for (int idx = lane; idx < nslots * cpr; idx += kWave) {
        const int a = idx / cpr, c = idx - a * cpr;
        const Slot sl = s_slots[a];
        const bool is_shared = sl.e < 0;
        const int e = is_shared ? 0 : sl.e;
        const W4 D = is_shared ? shared.down : routed.down;
        u32x4 cd[kDnRowsPerWave];
        float sd[kDnRowsPerWave], bd[kDnRowsPerWave];
#pragma unroll
        for (int r = 0; r < kDnRowsPerWave; ++r) {
            const size_t row = (size_t)e * H + (n0 + r);
            cd[r] = load_u32x4(D.codes + row * (I / 2) + c * 16);
            const size_t gi = row * ngroups + (c >> 1);
            sd[r] = bf16_to_f32(D.scales[gi]);
            bd[r] = bf16_to_f32(D.biases[gi]) - 128.0f * sd[r];
        }
        for (int i = 0; i < sl.cnt; ++i) {
            const int hrow = sl.off + i;
            int t;
            float w;
            if (is_shared) { t = i; w = 1.0f; }
            else { const int f = min(max(perm[hrow], 0), T * k - 1); t = f / k; w = topk_w[f]; }
            uint32_t xi[16];
            float hs;
            load_interleaved32(h + (size_t)hrow * I + c * 32, xi, hs);
#pragma unroll
            for (int r = 0; r < kDnRowsPerWave; ++r) {
                const float v = w * fmaf(sd[r], dot32_magic(cd[r], xi), bd[r] * hs);
#pragma unroll
                for (int tt = 0; tt < TMAX; ++tt) acc[r][tt] += (tt == t) ? v : 0.f;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kDnRowsPerWave; ++r)
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t >= T) break;
            const float v = wave_sum(acc[r][t]);
            if (lane == 0) out[(size_t)t * H + n0 + r] = (uint16_t)f32_to_bf16(v);
        }
}

template <int TMAX>
static hipError_t decode_t(const ForwardArgs& a, hipStream_t st, KernelTimer& tm) {
    const int max_slots = min(a.E, a.T * a.k) + (a.has_shared ? 1 : 0);
    dim3 g1(max_slots, a.I / kGuRowsPerBlock);
    tm.before();
    hipLaunchKernelGGL(k_decode_gateup<TMAX>, g1, dim3(256), 0, st, a.x, a.T, a.H, a.I, a.E, a.k,
                       a.routed, a.shared, a.has_shared, a.offsets, a.perm, a.ws_h);
    tm.after();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    hipLaunchKernelGGL(k_decode_down<TMAX>, dim3(a.H / kDnRowsPerBlock), dim3(256), 0, st, a.T,
                       a.H, a.I, a.E, a.k, a.routed, a.shared, a.has_shared, a.topk_w, a.offsets,
                       a.perm, a.ws_h, a.out);
    tm.after();
    return hipGetLastError();
}

hipError_t launch_forward_decode(const ForwardArgs& a, hipStream_t st, KernelTimer& tm) {
    if (a.T <= 1) return decode_t<1>(a, st, tm);
    if (a.T <= 2) return decode_t<2>(a, st, tm);
    if (a.T <= 4) return decode_t<4>(a, st, tm);
    return decode_t<8>(a, st, tm);
}

}  // namespace moe_w4
