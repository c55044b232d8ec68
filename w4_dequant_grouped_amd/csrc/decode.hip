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
//   k_decode_gateup: (slot, 8 rows of I) per workgroup -> h = silu(g) * u (bf16)
//   k_decode_down:   8 output rows per workgroup, every slot -> out (bf16)
// and the single-call block for T <= 4 (route + forward in three launches,
// described above k_decode_logits_shared).
// A slot is the shared expert (first: it needs no routing, so its workgroups
// start streaming at once) or an expert with a non-empty segment (ascending id).
// Both kernels read the routing from the device; the grid depends only on T.
#include "device.h"
#include "gemv.h"
#include "kernels.h"
#include "topk.h"

namespace moe_w4 {

constexpr int kMaxSlots = kDecodeMaxT * 16 + 1;

struct Slot {
    int e;      // expert id, or -1 for the shared expert
    int off;    // first h row of the slot
    int cnt;    // rows (tokens) in the slot
};

// Lane l owns experts [l*per, l*per + per), per = ceil(E / 64) <= 16: it loads
// their offsets in one go (one memory round trip for the whole scan), flags the
// non-empty segments and gets an exclusive prefix count over the lanes.
// Segments are clipped to the T*k routed rows, so malformed offsets cannot send
// a row index out of range.
struct ActiveScan {
    int lo[17];        // clipped offsets of the lane's experts (lo[j]..lo[j+1])
    int first;         // first expert of the lane
    int per;           // experts per lane
    int count;         // non-empty segments of the lane
    int before;        // non-empty segments of lower lanes
    int total;         // non-empty segments overall
};

__device__ __forceinline__ void scan_active(const int32_t* __restrict__ offsets, int E, int T, int k,
                                            int lane, ActiveScan& a) {
    const int lim = T * k;
    a.per = (E + kWave - 1) / kWave;
    a.first = lane * a.per;
#pragma unroll
    for (int j = 0; j < 17; ++j) {
        const int e = a.first + j;
        const int v = (j <= a.per && e <= E) ? offsets[min(e, E)] : lim;
        a.lo[j] = min(max(v, 0), lim);
    }
    int c = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < a.per && a.first + j < E) {
            a.lo[j + 1] = max(a.lo[j + 1], a.lo[j]);
            c += (a.lo[j + 1] > a.lo[j]) ? 1 : 0;
        }
    }
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    a.count = c;
    a.before = incl - c;
    a.total = __shfl(incl, kWave - 1, kWave);
}

// Slot list: the shared expert first (it needs no routing), then the experts
// with a non-empty segment in ascending id.  Built by wavefront 0.
__device__ __forceinline__ void build_slots(const int32_t* __restrict__ offsets, int E, int T, int k,
                                            int has_shared, Slot* s_slots, int* s_n, int lane) {
    ActiveScan a;
    scan_active(offsets, E, T, k, lane, a);
    const int base = has_shared ? 1 : 0;
    if (has_shared && lane == 0) s_slots[0] = Slot{-1, T * k, T};
    int pos = base + a.before;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < a.per && a.first + j < E && a.lo[j + 1] > a.lo[j]) {
            if (pos < kMaxSlots) s_slots[pos] = Slot{a.first + j, a.lo[j], min(a.lo[j + 1] - a.lo[j], T)};
            ++pos;
        }
    }
    if (lane == 0) *s_n = min(base + a.total, kMaxSlots);
}

// Slot table written by the routing kernel of the decode block (1 + 5 T k
// words): [0] = n; (expert, first h row, rows) of the i-th selected expert in
// ascending id at 1 + 3 i, i < n; (token, weight bits) of routed h row p at
// slot_rows_at(T, k) + 2 p, p < T k.  Every read is clamped to the ranges the
// kernels assume.
__device__ __forceinline__ int slot_rows_at(int T, int k) { return 1 + 3 * T * k; }
__device__ __forceinline__ int slot_count(const int32_t* __restrict__ table, int T, int k, int base) {
    return min(max(table[0], 0), min(T * k, kMaxSlots - base));
}
__device__ __forceinline__ int slot_expert(const int32_t* __restrict__ table, int i, int E) {
    return min(max(table[1 + 3 * i], 0), E - 1);
}

// The idx-th non-empty expert (ascending id), found by one wavefront;
// Slot{-2, 0, 0} if there are fewer.
__device__ __forceinline__ Slot find_slot(const int32_t* __restrict__ offsets, int E, int T, int k,
                                          int idx, int lane) {
    ActiveScan a;
    scan_active(offsets, E, T, k, lane, a);
    if (idx >= a.total) return Slot{-2, 0, 0};
    const bool mine = idx >= a.before && idx < a.before + a.count;
    Slot r{0, 0, 0};
    if (mine) {
        int n = idx - a.before;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < a.per && a.first + j < E && a.lo[j + 1] > a.lo[j]) {
                if (n == 0) r = Slot{a.first + j, a.lo[j], min(a.lo[j + 1] - a.lo[j], T)};
                --n;
            }
        }
    }
    const int src = __ffsll((long long)__ballot(mine)) - 1;
    return Slot{__shfl(r.e, src, kWave), __shfl(r.off, src, kWave), __shfl(r.cnt, src, kWave)};
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU
// ---------------------------------------------------------------------------
// Weight rows per wavefront: 2 for every row count.  A decode gate/up wavefront
// is one memory round trip plus its dot products and one wavefront reduction
// per row; two rows halve that tail against four, with twice the workgroups
// (measured per layer-call: T=1 21.1 -> 18.7 us, T=2 28.2 -> 25.1, T=4
// 44.7 -> 42.6; one row was slower again at T=1, 20.2 us, with every extra
// workgroup repeating the top-k).
template <int TMAX>
constexpr int gu_rows_per_wave() { return 2; }
template <int TMAX>
constexpr int gu_rows_per_block() { return 4 * gu_rows_per_wave<TMAX>(); }

// One token row: rows n0 .. n0+R-1 of gate and up of expert e,
// h[hrow0][n0 + r] = silu(gate . x) * (up . x), bf16.  One wavefront; every lane
// loads its own slice of x next to its weights (one memory round trip).
__device__ __forceinline__ void gateup_rows_one(const uint16_t* __restrict__ x, int H, int I,
                                                const W4& G, const W4& U, int e, int n0, int tok,
                                                int hrow0, uint16_t* __restrict__ h, int lane) {
    constexpr int R = gu_rows_per_wave<1>();
    const int ngroups = H / kGroup;
    const int nchunks = H / 32;
    float ag[R], au[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { ag[r] = 0.f; au[r] = 0.f; }

    for (int c = lane; c < nchunks; c += kWave) {
        u32x4 cg[R], cu[R];
        uint32_t sg[R], bg[R], su[R], bu[R];
        u32x4 xv[4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t row = (size_t)e * I + (n0 + r);
            cg[r] = load_u32x4(G.codes + row * (H / 2) + c * 16);
            cu[r] = load_u32x4(U.codes + row * (H / 2) + c * 16);
            const size_t gi = row * ngroups + (c >> 1);
            sg[r] = G.scales[gi];
            bg[r] = G.biases[gi];
            su[r] = U.scales[gi];
            bu[r] = U.biases[gi];
        }
        load64(x + (size_t)tok * H + c * 32, xv);
        uint32_t xi[16];
        float xs;
        interleave32(xv, xi, xs);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float s0 = bf16_to_f32(sg[r]), s1 = bf16_to_f32(su[r]);
            ag[r] += fmaf(s0, dot32_magic(cg[r], xi), (bf16_to_f32(bg[r]) - 128.0f * s0) * xs);
            au[r] += fmaf(s1, dot32_magic(cu[r], xi), (bf16_to_f32(bu[r]) - 128.0f * s1) * xs);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float g = wave_sum(ag[r]);
        const float u = wave_sum(au[r]);
        if (lane == r) h[(size_t)hrow0 * I + n0 + r] = (uint16_t)f32_to_bf16(silu(g) * u);
    }
}

// Several token rows.  The four wavefronts of a workgroup work on the same
// slot, hence the same token rows: x is staged once per workgroup in LDS, 64
// chunks of 32 values (2048 of K) at a time, already interleaved, with each
// chunk's sum.  [t][quarter][chunk] order keeps a wavefront's 16-byte reads
// consecutive.
constexpr int kXChunks = 64;
template <int TMAX>
struct XStage {
    u32x4 v[TMAX][4][kXChunks];
    float s[TMAX][kXChunks];
};

// An empty asm that claims to modify v: values computed from v before it cannot
// be reused after it.  The token loop uses it so that the compiler recomputes
// the codes' magic pairs per token (two bit operations each) instead of holding
// all of them in registers across the loop.
__device__ __forceinline__ void opaque(u32x4& v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

template <int TMAX>
__device__ __forceinline__ void gateup_rows_multi(const uint16_t* __restrict__ x, int H, int I,
                                                  const W4& G, const W4& U, int e, int n0, int cnt,
                                                  const int (&tok)[TMAX], int hrow0,
                                                  uint16_t* __restrict__ h, int lane, int wave,
                                                  XStage<TMAX>& sx) {
    constexpr int R = gu_rows_per_wave<TMAX>();
    constexpr int NQ = (TMAX + 3) / 4;          // token rows staged per wavefront
    const int ngroups = H / kGroup;
    const int nchunks = H / 32;
    float ag[R][TMAX], au[R][TMAX];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < TMAX; ++i) { ag[r][i] = 0.f; au[r][i] = 0.f; }

    for (int cb = 0; cb < nchunks; cb += kXChunks) {
        const int c = cb + lane;
        const bool own = c < nchunks;
        const int cl = own ? c : nchunks - 1;   // in-bounds address for idle lanes
        // x of the token rows this wavefront stages (t = wave, wave + 4): issued
        // first, since it is consumed first
        u32x4 xv[NQ][4];
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            if ((t & 3) == wave && t < cnt) load64(x + (size_t)tok[t] * H + cl * 32, xv[t >> 2]);
        u32x4 cg[R], cu[R];
        uint32_t sg[R], bg[R], su[R], bu[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t row = (size_t)e * I + (n0 + r);
            cg[r] = load_u32x4(G.codes + row * (H / 2) + cl * 16);
            cu[r] = load_u32x4(U.codes + row * (H / 2) + cl * 16);
            const size_t gi = row * ngroups + (cl >> 1);
            sg[r] = G.scales[gi];
            bg[r] = G.biases[gi];
            su[r] = U.scales[gi];
            bu[r] = U.biases[gi];
        }
        if (cb > 0) __syncthreads();            // the previous block's readers are done
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if ((t & 3) == wave && t < cnt) {
                uint32_t xi[16];
                float xs;
                interleave32(xv[t >> 2], xi, xs);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    sx.v[t][b][lane] = u32x4{xi[4 * b], xi[4 * b + 1], xi[4 * b + 2], xi[4 * b + 3]};
                sx.s[t][lane] = xs;
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t >= cnt) break;
#pragma unroll
            for (int r = 0; r < R; ++r) { opaque(cg[r]); opaque(cu[r]); }
            uint32_t xi[16];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const u32x4 q = sx.v[t][b][lane];
                xi[4 * b] = q.x; xi[4 * b + 1] = q.y; xi[4 * b + 2] = q.z; xi[4 * b + 3] = q.w;
            }
            const float xs = sx.s[t][lane];
            if (own) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float s0 = bf16_to_f32(sg[r]), s1 = bf16_to_f32(su[r]);
                    ag[r][t] += fmaf(s0, dot32_magic(cg[r], xi), (bf16_to_f32(bg[r]) - 128.0f * s0) * xs);
                    au[r][t] += fmaf(s1, dot32_magic(cu[r], xi), (bf16_to_f32(bu[r]) - 128.0f * s1) * xs);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
        if (i >= cnt) break;
        const int hrow = hrow0 + i;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float g = wave_sum(ag[r][i]);
            const float u = wave_sum(au[r][i]);
            if (lane == r) h[(size_t)hrow * I + n0 + r] = (uint16_t)f32_to_bf16(silu(g) * u);
        }
    }
}

// Rows n0 .. n0 + R - 1 of gate and up of expert e for the cnt token rows
// tok[0..cnt): h[hrow0 + i][n0 + r] = silu(gate . x_tok[i]) * (up . x_tok[i]).
// All four wavefronts of the workgroup must call it with the same slot.
template <int TMAX>
__device__ __forceinline__ void gateup_rows(const uint16_t* __restrict__ x, int H, int I,
                                            const W4& G, const W4& U, int e, int n0, int cnt,
                                            const int (&tok)[TMAX], int hrow0,
                                            uint16_t* __restrict__ h, int lane, int wave) {
    if constexpr (TMAX == 1) {
        gateup_rows_one(x, H, I, G, U, e, n0, tok[0], hrow0, h, lane);
    } else {
        __shared__ XStage<TMAX> s_x;
        gateup_rows_multi<TMAX>(x, H, I, G, U, e, n0, cnt, tok, hrow0, h, lane, wave, s_x);
    }
}

template <int TMAX>
__global__ __launch_bounds__(256) void k_decode_gateup(
    const uint16_t* __restrict__ x, int T, int H, int I, int E, int k,
    W4Set routed, W4Set shared, int has_shared,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    uint16_t* __restrict__ h) {
    __shared__ Slot s_slot;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    Slot sl;
    if (has_shared && blockIdx.x == 0) {
        sl = Slot{-1, T * k, T};                 // no dependence on the routing
    } else {
        if (wave == 0) {
            const Slot f = find_slot(offsets, E, T, k, blockIdx.x - (has_shared ? 1 : 0), lane);
            if (lane == 0) s_slot = f;
        }
        __syncthreads();
        sl = s_slot;
        if (sl.e < -1) return;                   // fewer active experts than blocks
    }
    const bool is_shared = sl.e < 0;
    const int e = is_shared ? 0 : sl.e;
    const W4 G = is_shared ? shared.gate : routed.gate;
    const W4 U = is_shared ? shared.up : routed.up;

    // token of each row of the slot
    int tok[TMAX];
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
        tok[i] = 0;
        if (TMAX > 1 && i < sl.cnt)
            tok[i] = is_shared ? i : min(max(perm[sl.off + i], 0), T * k - 1) / k;
    }
    const int n0 = blockIdx.y * gu_rows_per_block<TMAX>() + wave * gu_rows_per_wave<TMAX>();
    gateup_rows<TMAX>(x, H, I, G, U, e, n0, sl.cnt, tok, sl.off, h, lane, wave);
}

// ---------------------------------------------------------------------------
// down + weighted combine
// ---------------------------------------------------------------------------
constexpr int kDnRowsPerWave = 2;
constexpr int kDnRowsPerBlock = 4 * kDnRowsPerWave;
constexpr int kDnUnroll = 4;     // (slot, 32-code chunk) items per lane in one batch of loads
constexpr int kDnLdsI = 512;     // h is staged in LDS when I <= this
constexpr int kDnThreads = 256;  // threads per down workgroup

// h rows of T <= TMAX tokens: T*k routed + T shared, k <= 16
template <int TMAX>
constexpr int dn_rows() { return TMAX * (kMaxTopK + 1); }

// One batch of down-weight loads: kDnUnroll items per lane.
struct DnBatch {
    u32x4 c[kDnUnroll][kDnRowsPerWave];
    uint32_t s[kDnUnroll][kDnRowsPerWave], b[kDnUnroll][kDnRowsPerWave];
    int slot[kDnUnroll], cc[kDnUnroll];   // slot (-1: no item) and chunk
};

// Rows n0, n0+1 per wavefront.  A lane's items are (slot, chunk) pairs; each is
// dotted with every token row of its slot.  Before the item loop, h (all
// threads), the slot list (wavefront 0) and each h row's token and weight
// (wavefront 1) go to LDS in parallel, so that no batch of weight loads waits
// on a dependent global read, and the next batch is in flight while the
// current one is used.  Given the routing kernel's slot table, the first
// batch's experts are read from it directly and its weight loads are issued
// before that staging, and the rows' tokens and weights come from the table in
// one round trip.  HLDS: h staged in LDS (I <= kDnLdsI), else read from global
// memory.  A compile-time choice: a global read inside the item loop would make
// every iteration wait for the next batch's loads too.
template <int TMAX, bool HLDS, bool kTable>
__global__ __launch_bounds__(kDnThreads) void k_decode_down(
    int T, int H, int I, int E, int k, W4Set routed, W4Set shared, int has_shared,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const uint16_t* __restrict__ h,
    uint16_t* __restrict__ out, const int32_t* __restrict__ slot_table) {
    constexpr int HR = dn_rows<TMAX>();
    __shared__ Slot s_slots[kMaxSlots];
    __shared__ int s_n;
    __shared__ int s_rt[HR];          // token of each h row
    __shared__ float s_rw[HR];        // its routing weight (1 for the shared expert)
    __shared__ __attribute__((aligned(16))) uint16_t s_h[HLDS ? HR * kDnLdsI : 8];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int hrows = T * k + T;
    const int base = has_shared ? 1 : 0;
    const int n0 = blockIdx.x * kDnRowsPerBlock + wave * kDnRowsPerWave;
    const int cpr = I / 32;            // 32-code chunks per down row
    const int ngroups = I / kGroup;
    constexpr int kStep = kWave * kDnUnroll;
    // ex[u]: expert of item u's slot, negative for the shared expert; items past
    // the end load chunk 0 of an in-bounds expert (never used)
    auto load = [&](DnBatch& B, int first, int nitems, const int (&ex)[kDnUnroll]) {
#pragma unroll
        for (int u = 0; u < kDnUnroll; ++u) {
            const int idx = first + u * kWave + lane;
            const bool ok = idx < nitems;
            const int a = ok ? idx / cpr : 0;
            B.slot[u] = ok ? a : -1;
            B.cc[u] = ok ? idx - a * cpr : 0;
            const bool is_shared = ex[u] < 0;
            const int e = is_shared ? 0 : ex[u];
            const W4 D = is_shared ? shared.down : routed.down;
#pragma unroll
            for (int r = 0; r < kDnRowsPerWave; ++r) {
                const size_t row = (size_t)e * H + (n0 + r);
                B.c[u][r] = load_u32x4(D.codes + row * (I / 2) + B.cc[u] * 16);
                const size_t gi = row * ngroups + (B.cc[u] >> 1);
                B.s[u][r] = D.scales[gi];
                B.b[u][r] = D.biases[gi];
            }
        }
    };
    auto load_lds = [&](DnBatch& B, int first, int nitems) {
        int ex[kDnUnroll];
#pragma unroll
        for (int u = 0; u < kDnUnroll; ++u) {
            const int idx = first + u * kWave + lane;
            ex[u] = s_slots[idx < nitems ? idx / cpr : 0].e;
        }
        load(B, first, nitems, ex);
    };
    DnBatch cur, nxt;
    // h: all of this thread's loads first (unconditional, index clamped; T >= 1
    // here, so h is not empty), the LDS writes later: one round trip
    constexpr int kPer = HLDS ? (HR * kDnLdsI / 8 + kDnThreads - 1) / kDnThreads : 1;
    const int n16 = hrows * I / 8;
    u32x4 hv[kPer];
    auto load_h = [&]() {
#pragma unroll
        for (int q = 0; q < kPer; ++q)
            hv[q] = reinterpret_cast<const u32x4*>(h)[min((int)threadIdx.x + q * kDnThreads, n16 - 1)];
    };
    auto store_h = [&]() {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int i = threadIdx.x + q * kDnThreads;
            if (i < n16) reinterpret_cast<u32x4*>(s_h)[i] = hv[q];
        }
    };
    int nitems;
    if constexpr (kTable) {
        // Straight-line, every read issued before any wait that the weights
        // would hold up (loads complete in issue order): the table entries of
        // the first batch's items, of every slot and of every routed h row (one
        // lane each per pass of 64), the count; then the first batch's weights;
        // then h; then the LDS writes.
        constexpr int kP = (TMAX * kMaxTopK + TMAX + kWave - 1) / kWave;   // passes of 64 slots or rows
        static_assert(kP <= 2, "table reads below");
        int ex[kDnUnroll];
#pragma unroll
        for (int u = 0; u < kDnUnroll; ++u) {
            const int a = (u * kWave + lane) / cpr;
            ex[u] = slot_table[1 + 3 * min(max(a - base, 0), T * k - 1)];
        }
        // lane i of pass p reads words 3 i .. 3 i + 3 for slot i = 64 p + lane
        // (clamped into the table), and in pass 0 lane 0 the count (a vector
        // read, so that no scalar wait comes before the other reads)
        int c0 = 0, se[kP], so[kP], sc[kP], rt[kP], rw[kP];
#pragma unroll
        for (int p = 0; p < kP; ++p) {
            const int i = min(kWave * p + lane, T * k - 1);
            if (p == 0) c0 = slot_table[3 * i];
            se[p] = slot_table[1 + 3 * i];
            so[p] = slot_table[2 + 3 * i];
            sc[p] = slot_table[3 + 3 * i];
            rt[p] = slot_table[slot_rows_at(T, k) + 2 * i];
            rw[p] = slot_table[slot_rows_at(T, k) + 2 * i + 1];
        }
        // an empty asm that takes every table value: all the reads above are
        // issued before it and no use of one is moved above it (one wait)
        static_assert(kDnUnroll == 4, "operands below");
        if constexpr (kP == 1) {
            asm volatile("" : "+v"(c0), "+v"(se[0]), "+v"(so[0]), "+v"(sc[0]), "+v"(rt[0]), "+v"(rw[0]),
                              "+v"(ex[0]), "+v"(ex[1]), "+v"(ex[2]), "+v"(ex[3]));
        } else {
            asm volatile("" : "+v"(c0), "+v"(se[0]), "+v"(so[0]), "+v"(sc[0]), "+v"(rt[0]), "+v"(rw[0]),
                              "+v"(se[kP - 1]), "+v"(so[kP - 1]), "+v"(sc[kP - 1]), "+v"(rt[kP - 1]),
                              "+v"(rw[kP - 1]), "+v"(ex[0]), "+v"(ex[1]), "+v"(ex[2]), "+v"(ex[3]));
        }
        const int nsel = min(max(__builtin_amdgcn_readfirstlane(c0), 0), min(T * k, kMaxSlots - base));
        nitems = (base + nsel) * cpr;
#pragma unroll
        for (int u = 0; u < kDnUnroll; ++u) {
            const int a = (u * kWave + lane) / cpr;
            ex[u] = a < base ? -1 : min(max(ex[u], 0), E - 1);
        }
        load(cur, 0, nitems, ex);
        if constexpr (HLDS) {
            load_h();
            store_h();
        }
        if (wave == 0) {
            if (has_shared && lane == 0) s_slots[0] = Slot{-1, T * k, T};
#pragma unroll
            for (int p = 0; p < kP; ++p) {
                const int i = kWave * p + lane;
                if (i < nsel) {
                    const int off = min(max(so[p], 0), T * k);
                    s_slots[base + i] = Slot{min(max(se[p], 0), E - 1), off, min(max(sc[p], 0), min(T, T * k - off))};
                }
            }
            if (lane == 0) s_n = base + nsel;
        } else if (wave == 1) {
#pragma unroll
            for (int p = 0; p < kP; ++p) {
                const int r = kWave * p + lane;
                if (r < hrows) {
                    const bool routed_row = r < T * k;
                    s_rt[r] = routed_row ? min(max(rt[p], 0), T - 1) : r - T * k;
                    s_rw[r] = routed_row ? __int_as_float(rw[p]) : 1.0f;
                }
            }
        }
        __syncthreads();
    } else {
        if constexpr (HLDS) {
            load_h();
            store_h();
        }
        if (wave == 0) {
            build_slots(offsets, E, T, k, has_shared, s_slots, &s_n, lane);
        } else if (wave == 1) {
            for (int r = lane; r < hrows; r += kWave) {
                int t;
                float w;
                if (r >= T * k) {
                    t = r - T * k;
                    w = 1.0f;
                } else {
                    const int f = min(max(perm[r], 0), T * k - 1);
                    t = f / k;
                    w = topk_w[f];
                }
                s_rt[r] = t;
                s_rw[r] = w;
            }
        }
        __syncthreads();
        nitems = s_n * cpr;
        load_lds(cur, 0, nitems);
    }
    float acc[kDnRowsPerWave][TMAX];
#pragma unroll
    for (int r = 0; r < kDnRowsPerWave; ++r)
#pragma unroll
        for (int t = 0; t < TMAX; ++t) acc[r][t] = 0.f;
    for (int first = 0; first < nitems; first += kStep) {
        // next batch in flight during this one; none past the end (its loads
        // would still be waited for before the kernel's last instructions)
        const bool more = first + kStep < nitems;
        if (more) load_lds(nxt, first + kStep, nitems);
#pragma unroll
        for (int u = 0; u < kDnUnroll; ++u) {
            if (cur.slot[u] < 0) continue;
            const Slot sl = s_slots[cur.slot[u]];
            for (int i = 0; i < sl.cnt; ++i) {
                const int hrow = sl.off + i;
                const int t = s_rt[hrow];
                const float w = s_rw[hrow];
                u32x4 hv[4];
                if constexpr (HLDS) {
                    const u32x4* q = reinterpret_cast<const u32x4*>(s_h + (size_t)hrow * I + cur.cc[u] * 32);
#pragma unroll
                    for (int b = 0; b < 4; ++b) hv[b] = q[b];
                } else {
                    load64(h + (size_t)hrow * I + cur.cc[u] * 32, hv);
                }
                uint32_t xi[16];
                float hs;
                interleave32(hv, xi, hs);
#pragma unroll
                for (int r = 0; r < kDnRowsPerWave; ++r) {
                    const float s0 = bf16_to_f32(cur.s[u][r]);
                    const float v = w * fmaf(s0, dot32_magic(cur.c[u][r], xi),
                                             (bf16_to_f32(cur.b[u][r]) - 128.0f * s0) * hs);
#pragma unroll
                    for (int tt = 0; tt < TMAX; ++tt) acc[r][tt] += (tt == t) ? v : 0.f;
                }
            }
        }
        if (!more) break;
        cur = nxt;
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
    dim3 g1(max_slots, a.I / gu_rows_per_block<TMAX>());
    tm.before();
    tm.launch(k_decode_gateup<TMAX>, g1, dim3(256), 0, st, a.x, a.T, a.H, a.I, a.E, a.k,
                       a.routed, a.shared, a.has_shared, a.offsets, a.perm, a.ws_h);
    tm.after();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    tm.launch(a.I <= kDnLdsI ? k_decode_down<TMAX, true, false> : k_decode_down<TMAX, false, false>,
              dim3(a.H / kDnRowsPerBlock), dim3(kDnThreads), 0, st, a.T, a.H, a.I, a.E, a.k, a.routed,
              a.shared, a.has_shared, a.topk_w, a.offsets, a.perm, a.ws_h, a.out, nullptr);
    tm.after();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Route + forward of decode rows in three launches (moe_w4_block)
// ---------------------------------------------------------------------------
// Launch 1: router logits (a wavefront per expert) and the shared expert's
//   gate/up -- both need only x, so their bytes stream together.
// Launch 2: every workgroup reads the T x E logits and repeats the (cheap)
//   top-k; the workgroup of the last column writes the routing outputs and the
//   slot table and runs no expert rows.  Workgroup (s, y) runs rows
//   8y .. 8y+7 of gate/up of the s-th selected expert (ascending id); at T = 1
//   each wavefront selects on its own and needs no grouping.  There is no
//   "last workgroup" hand-off inside the router: the kernel boundary is the
//   only grid-wide dependency between the logits and the expert weights.
// Launch 3: k_decode_down over the shared expert and the selected experts.

template <int TMAX>
__global__ __launch_bounds__(256) void k_decode_logits_shared(DecodeBlockArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int T = a.T, H = a.H, E = a.E;
    const int nlog = (E + 3) / 4;
    if ((int)blockIdx.x < nlog) {
        const int e = blockIdx.x * 4 + wave;
        if (e >= E) return;
        float acc[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) acc[t] = 0.f;
        const float* wrow = a.Wr + (size_t)e * H;
        for (int h0 = 0; h0 < H; h0 += kWave * 4 * 8) {
            float4 wv[8];
            u32x2 xv[8][TMAX];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int hh = h0 + (u * kWave + lane) * 4;
                const bool ok = hh < H;
                wv[u] = ok ? *reinterpret_cast<const float4*>(wrow + hh) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < TMAX; ++t)
                    xv[u][t] = (ok && t < T) ? *reinterpret_cast<const u32x2*>(a.x + (size_t)t * H + hh)
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
        const float bias = a.br ? a.br[e] : 0.f;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t >= T) break;
            const float sum = wave_sum(acc[t]);
            if (lane == 0) a.logits[t * E + e] = sum + bias;
        }
    } else {
        int tok[TMAX];
#pragma unroll
        for (int i = 0; i < TMAX; ++i) tok[i] = i;
        const int n0 = (blockIdx.x - nlog) * gu_rows_per_block<TMAX>() + wave * gu_rows_per_wave<TMAX>();
        gateup_rows<TMAX>(a.x, H, a.I, a.shared.gate, a.shared.up, 0, n0, T, tok, T * a.k, a.h, lane, wave);
    }
}

template <int TMAX, int EPL>
__global__ __launch_bounds__(256) void k_decode_route_gateup(DecodeBlockArgs a) {
    constexpr int N = TMAX * kMaxTopK;            // (token, slot) entries at most
    __shared__ float s_w[N];
    __shared__ uint64_t s_mask[TMAX][EPL];        // chosen experts of each token
    __shared__ int s_ptok[N];
    __shared__ int s_u[N], s_uoff[N], s_ucnt[N];
    __shared__ int s_nu;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int T = a.T, E = a.E, k = a.k;
    // the workgroup past the last slot column writes the routing outputs and
    // runs no expert rows (its other rows have nothing to do)
    const bool writer = blockIdx.x == gridDim.x - 1;
    if (writer && blockIdx.y != 0) return;

    if constexpr (TMAX == 1) {
        if (!writer) {
            // One row: every selected expert has exactly one h row, the rank of its id
            // among the chosen, so no grouping is needed.  Each wavefront selects on
            // its own (no barrier, no LDS) and streams its expert's rows as soon as it
            // knows it.
            float vals[EPL];
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane + kWave * j;
                vals[j] = (e < E) ? a.logits[e] : -INFINITY;
            }
            const int slot = blockIdx.x;               // grid.x = min(E, k) + 1: slot < k
            const int e = wave_topk_nth<EPL>(vals, E, k, lane, slot);
            const int tok1[1] = {0};
            const int n0 = blockIdx.y * gu_rows_per_block<1>() + wave * gu_rows_per_wave<1>();
            gateup_rows<1>(a.x, a.H, a.I, a.routed.gate, a.routed.up, e, n0, 1, tok1, slot, a.h, lane, wave);
            return;
        }
    }

    // top-k of every token: wavefront t
    for (int t = wave; t < T; t += 4) {
        float vals[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + kWave * j;
            vals[j] = (e < E) ? a.logits[t * E + e] : -INFINITY;
        }
        // the writer also keeps the weights in LDS for the row table; the other
        // workgroups need only the selection masks
        wave_topk_select<EPL>(vals, E, k, lane, writer ? a.ids + t * k : nullptr,
                              writer ? a.tw + t * k : nullptr, nullptr, writer ? s_w + t * k : nullptr,
                              &s_mask[t][0]);
    }
    __syncthreads();
    // grouping by wavefront 0 from the selection masks: lane l handles experts
    // e = l + 64 j.  Entries of lower experts = popcounts of the masks below e;
    // entries of e from earlier tokens = mask bits of e in those tokens; the
    // rank of e among the selected experts = popcounts of the union below e;
    // e's slot within a token = that token's popcounts below e.
    if (wave == 0) {
        // all masks in registers (one LDS round trip), zero past T
        uint64_t mk[TMAX][EPL];
        int pre[TMAX][EPL];              // token t's chosen experts below 64 j
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            int run = 0;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                mk[t][j] = (t < T) ? s_mask[t][j] : 0ull;
                pre[t][j] = run;
                run += __builtin_popcountll(mk[t][j]);
            }
        }
        int nu = 0;
        int below_j = 0;                 // entries of experts < 64 j
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + kWave * j;
            uint64_t un = 0ull;
            int below = below_j, cnt = 0, tot_j = 0;
#pragma unroll
            for (int t = 0; t < TMAX; ++t) {
                un |= mk[t][j];
                below += bits_below(mk[t][j]);
                cnt += (int)((mk[t][j] >> lane) & 1ull);
                tot_j += __builtin_popcountll(mk[t][j]);
            }
            if (writer && e < E) {
                a.offsets[e] = below;
                a.counts[e] = cnt;
            }
            if (cnt > 0) {
                const int rank = nu + bits_below(un);
                s_u[rank] = e;
                s_uoff[rank] = below;
                s_ucnt[rank] = cnt;
                int before = 0;
#pragma unroll
                for (int t = 0; t < TMAX; ++t) {
                    if ((mk[t][j] >> lane) & 1ull) {
                        const int p = below + before;
                        s_ptok[p] = t;
                        if (writer) {
                            const int f = t * k + pre[t][j] + bits_below(mk[t][j]);
                            a.perm[p] = f;
                            a.slots[slot_rows_at(T, k) + 2 * p] = t;
                            a.slots[slot_rows_at(T, k) + 2 * p + 1] = __float_as_int(s_w[f]);
                        }
                        ++before;
                    }
                }
            }
            below_j += tot_j;
            nu += __builtin_popcountll(un);
        }
        if (writer && lane == 0) a.offsets[E] = T * k;
        if (lane == 0) s_nu = nu;
    }
    __syncthreads();
    if (writer) {                     // slot table for the down kernel
        const int nu = s_nu;
        for (int i = threadIdx.x; i < nu; i += blockDim.x) {
            a.slots[1 + 3 * i] = s_u[i];
            a.slots[2 + 3 * i] = s_uoff[i];
            a.slots[3 + 3 * i] = s_ucnt[i];
        }
        if (threadIdx.x == 0) a.slots[0] = nu;
        return;
    }
    const int nu = s_nu;
    const int slot = blockIdx.x;
    if (slot >= nu) return;
    const int cnt = min(s_ucnt[slot], T);
    int tok[TMAX];
#pragma unroll
    for (int i = 0; i < TMAX; ++i) tok[i] = s_ptok[s_uoff[slot] + min(i, cnt - 1)];
    const int n0 = blockIdx.y * gu_rows_per_block<TMAX>() + wave * gu_rows_per_wave<TMAX>();
    gateup_rows<TMAX>(a.x, a.H, a.I, a.routed.gate, a.routed.up, s_u[slot], n0, cnt, tok,
                      s_uoff[slot], a.h, lane, wave);
}

template <int TMAX, int EPL>
static hipError_t block_decode_t(const DecodeBlockArgs& a, hipStream_t st, KernelTimer& tm) {
    const int nlog = (a.E + 3) / 4;
    const int nsh = a.has_shared ? a.I / gu_rows_per_block<TMAX>() : 0;
    tm.before();
    tm.launch(k_decode_logits_shared<TMAX>, dim3(nlog + nsh), dim3(256), 0, st, a);
    tm.after();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    tm.launch((k_decode_route_gateup<TMAX, EPL>),
                       dim3(min(a.E, a.T * a.k) + 1, a.I / gu_rows_per_block<TMAX>()), dim3(256), 0, st, a);
    tm.after();
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    tm.launch(a.I <= kDnLdsI ? k_decode_down<TMAX, true, true> : k_decode_down<TMAX, false, true>,
              dim3(a.H / kDnRowsPerBlock), dim3(kDnThreads), 0, st, a.T, a.H, a.I, a.E, a.k, a.routed,
              a.shared, a.has_shared, a.tw, a.offsets, a.perm, a.h, a.out, a.slots);
    tm.after();
    return hipGetLastError();
}

template <int TMAX>
static hipError_t block_decode_e(const DecodeBlockArgs& a, hipStream_t st, KernelTimer& tm) {
    if (a.E <= 256) return block_decode_t<TMAX, 4>(a, st, tm);
    if (a.E <= 512) return block_decode_t<TMAX, 8>(a, st, tm);
    return block_decode_t<TMAX, 16>(a, st, tm);
}

hipError_t launch_block_decode(const DecodeBlockArgs& a, hipStream_t st, KernelTimer& tm) {
    static_assert(kBlockDecodeMaxT == 4, "instantiations below");
    switch (a.T) {
        case 1: return block_decode_e<1>(a, st, tm);
        case 2: return block_decode_e<2>(a, st, tm);
        case 3: return block_decode_e<3>(a, st, tm);
        case 4: return block_decode_e<4>(a, st, tm);
        default: return hipErrorInvalidValue;     // the host serves larger T by route + forward
    }
}

hipError_t launch_forward_decode(const ForwardArgs& a, hipStream_t st, KernelTimer& tm) {
    switch (a.T) {
        case 1: return decode_t<1>(a, st, tm);
        case 2: return decode_t<2>(a, st, tm);
        case 3: return decode_t<3>(a, st, tm);
        case 4: return decode_t<4>(a, st, tm);
        case 5: return decode_t<5>(a, st, tm);
        default: return decode_t<8>(a, st, tm);
    }
}

}  // namespace moe_w4
