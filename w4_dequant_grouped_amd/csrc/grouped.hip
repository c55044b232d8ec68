// Prefill path of the W4 MoE block: grouped GEMMs on bf16 MFMA (gfx950).
//
// Expert GEMMs dominate prefill ("Perplexity's Lily brings fast local AI to Apple
// silicon Macs", section "Where the Engine Gains Speed": roughly 90% of prefill
// time), and the 4-bit weights are reconstructed inside the grouped GEMM one tile
// at a time, so no expanded weight array ever reaches memory (same section, and
// "Perplexity built an inference engine for one model, one chip", paragraph 3).
//
// Kernels (one stream, no host round trip; the tile list is derived on the device
// from the routing offsets):
//   k_grouped_gateup  per tile (segment, 128-row M-tile, N-tile of I): the rows'
//                     activations are gathered by token into LDS, the gate and up
//                     codes are loaded 128 bits per lane straight into registers,
//                     dequantised (w = c * s + b, fp32 FMA, RNE to bf16) into the
//                     MFMA B operand and multiplied on v_mfma_f32_16x16x32_bf16
//                     with fp32 accumulation; the epilogue applies SwiGLU and
//                     writes h (bf16) in expert-sorted row order.  It also clears
//                     the fp32 output accumulator.
//   k_grouped_down    same K-loop over h (rows contiguous per expert), epilogue
//                     scales each row by its routing weight and adds it into the
//                     token's fp32 accumulator row (atomic add).
//   k_finalize        accumulator -> bf16 output (round to nearest even).
// A segment is a routed expert's rows (offsets[e]..offsets[e+1], tokens via the
// permutation) or the shared expert's rows (all tokens, weight 1).  Persistent
// workgroups walk the tile list; consecutive N-tiles of one M-tile are given to
// workgroups on the same XCD (workgroup b runs on XCD b mod 8) so the gathered
// activations are fetched into that XCD's L2 once.
//
// MFMA operand layout used (16x16x32, wave64): lane l supplies A row l%16 and B
// column l%16, each with 8 k values for the k-slot group l/16; D element
// (4*(l/16)+i, l%16) is accumulator i of lane l.  A lane loads 32 consecutive
// codes of one weight row (k = 32*(l/16) .. +32 of a 128-wide K chunk); MFMA step
// j consumes its 8 codes 8j..8j+7, and the A operand is read from LDS at the same
// logical k, so both operands agree on the k order.
#include "device.h"
#include "kernels.h"

namespace moe_w4 {

constexpr int kBM = 128;               // rows per M-tile
constexpr int kMB = kBM / 16;          // 16-row MFMA blocks per M-tile
constexpr int kKC = 128;               // K per chunk (4 MFMA steps of 32)
constexpr int kARowBytes = kKC * 2;    // bf16 bytes of one A row per chunk
constexpr int kAStride = kARowBytes + 16;   // padded LDS row stride
constexpr int kMaxSeg = 1025;
constexpr int kThreads = 256;

struct TileCtx {
    int seg;        // segment index (E = shared)
    int e;          // expert index within its weight set
    int shared;     // 1 for the shared expert
    int m0;         // first row of the M-tile within the segment
    int rows;       // valid rows
    int hbase;      // h row of the segment's first row
};

// Rows of segment s, with the routed segments clipped to the T*k routed rows so
// malformed offsets cannot send a row index out of range.
__device__ __forceinline__ int seg_first(const int32_t* __restrict__ offsets, int s, int E, int T, int k) {
    return (s < E) ? min(max(offsets[s], 0), T * k) : T * k;
}
__device__ __forceinline__ int seg_count(const int32_t* __restrict__ offsets, int s, int E, int T, int k) {
    if (s >= E) return T;
    const int a = seg_first(offsets, s, E, T, k);
    const int b = min(max(offsets[s + 1], a), T * k);
    return b - a;
}

// Per-segment M-tile counts -> exclusive prefix in LDS; returns the total.
__device__ int build_mtile_prefix(const int32_t* __restrict__ offsets, int E, int T, int k,
                                  int has_shared, int* s_pre, int* s_tmp) {
    const int nseg = E + (has_shared ? 1 : 0);
    const int tid = threadIdx.x;
    // each thread sums a contiguous run of segments
    const int per = (nseg + kThreads - 1) / kThreads;
    const int s0 = min(tid * per, nseg), s1 = min(s0 + per, nseg);
    int local = 0;
    for (int s = s0; s < s1; ++s) local += (seg_count(offsets, s, E, T, k) + kBM - 1) / kBM;
    s_tmp[tid] = local;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
        const int v = (tid >= o) ? s_tmp[tid - o] : 0;
        __syncthreads();
        s_tmp[tid] += v;
        __syncthreads();
    }
    int run = s_tmp[tid] - local;
    for (int s = s0; s < s1; ++s) {
        s_pre[s] = run;                  // exclusive prefix
        run += (seg_count(offsets, s, E, T, k) + kBM - 1) / kBM;
    }
    if (tid == kThreads - 1) s_pre[nseg] = s_tmp[kThreads - 1];
    __syncthreads();
    return s_pre[nseg];
}

__device__ __forceinline__ TileCtx locate(int mt, const int* s_pre, int nseg, int E, int T, int k,
                                          const int32_t* __restrict__ offsets) {
    int lo = 0, hi = nseg - 1;           // last seg with s_pre[seg] <= mt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    TileCtx c;
    c.seg = lo;
    c.shared = (lo >= E);
    c.e = c.shared ? 0 : lo;
    c.m0 = (mt - s_pre[lo]) * kBM;
    c.rows = min(kBM, seg_count(offsets, lo, E, T, k) - c.m0);
    c.hbase = seg_first(offsets, lo, E, T, k);
    return c;
}

// tile index -> (M-tile, N-tile): the NT N-tiles of one M-tile go to workgroups
// with equal index mod 8 (one XCD)
__device__ __forceinline__ void tile_coords(int i, int NT, int& mt, int& nt) {
    mt = (i & 7) + 8 * (i / (8 * NT));
    nt = (i >> 3) % NT;
}

// Stage one K chunk of A (kBM rows x kKC bf16) into LDS.  row_ptr(r) gives the
// start of row r's chunk; rows >= rows are zero-filled.
template <class RowPtr>
__device__ __forceinline__ void stage_a(uint8_t* s_a, int rows, RowPtr row_ptr) {
    const int tid = threadIdx.x;
    const int r = tid >> 1;                // 2 threads per row, 128 bytes each
    const int half = tid & 1;
    u32x4 v[8];
    if (r < rows) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(row_ptr(r)) + half * 128;
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = load_u32x4(src + 16 * q);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = u32x4{0u, 0u, 0u, 0u};
    }
    uint8_t* dst = s_a + r * kAStride + half * 128;
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4*>(dst + 16 * q) = v[q];
}

// One K chunk of MFMAs: NMAT matrices x NBW 16-column blocks per wavefront.
template <int NMAT, int NBW>
__device__ __forceinline__ void mma_chunk(const uint8_t* s_a, int rows, int lane,
                                          const u32x4 (&codes)[NMAT][NBW],
                                          const float (&sc)[NMAT][NBW], const float (&bi)[NMAT][NBW],
                                          f32x4 (&acc)[kMB][NMAT][NBW]) {
    const int arow = lane & 15;
    const int acol = (lane >> 4) * 64;     // byte offset of the lane's 32 k values
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bf16x8 b[NMAT][NBW];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const uint32_t d = (j == 0) ? codes[m][nb].x : (j == 1) ? codes[m][nb].y
                                 : (j == 2) ? codes[m][nb].z : codes[m][nb].w;
                b[m][nb] = dequant8(d, sc[m][nb], bi[m][nb]);
            }
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
            if (mb * 16 >= rows) break;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                s_a + (mb * 16 + arow) * kAStride + acol + j * 16);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    acc[mb][m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[m][nb],
                                                                            acc[mb][m][nb], 0, 0, 0);
        }
    }
}

// Load the lane's codes (128 bits) and group scale/bias for one K chunk.
__device__ __forceinline__ void load_b(const W4& W, int e, int N, int K, int n, int kc, int lane,
                                       u32x4& codes, float& s, float& b) {
    const size_t row = (size_t)e * N + n;
    codes = load_u32x4(W.codes + row * (K / 2) + (kc >> 1) + (lane >> 4) * 16);
    const size_t gi = row * (K / kGroup) + ((kc + (lane >> 4) * 32) / kGroup);
    s = bf16_to_f32(W.scales[gi]);
    b = bf16_to_f32(W.biases[gi]);
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU
// ---------------------------------------------------------------------------
template <int NBW>
__global__ __launch_bounds__(kThreads, 2) void k_grouped_gateup(
    const uint16_t* __restrict__ x, int T, int H, int I, int E, int k,
    W4Set routed, W4Set shared, int has_shared,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    uint16_t* __restrict__ h, float* __restrict__ acc_zero, long acc_elems) {
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kBM * kAStride];
    __shared__ int s_pre[kMaxSeg + 1];
    __shared__ int s_tmp[kThreads];
    __shared__ int s_tok[kBM];

    // clear the fp32 output accumulator for the down kernel
    for (long i = ((long)blockIdx.x * kThreads + threadIdx.x) * 4; i < acc_elems;
         i += (long)gridDim.x * kThreads * 4)
        *reinterpret_cast<float4*>(acc_zero + i) = float4{0.f, 0.f, 0.f, 0.f};

    const int nseg = E + (has_shared ? 1 : 0);
    const int n_mt = build_mtile_prefix(offsets, E, T, k, has_shared, s_pre, s_tmp);
    constexpr int BN = 4 * 16 * NBW;
    const int NT = I / BN;
    const int total = ((n_mt + 7) / 8) * 8 * NT;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    for (int i = blockIdx.x; i < total; i += gridDim.x) {
        int mt, nt;
        tile_coords(i, NT, mt, nt);
        if (mt >= n_mt) continue;
        const TileCtx c = locate(mt, s_pre, nseg, E, T, k, offsets);
        const W4Set& Wset = c.shared ? shared : routed;
        __syncthreads();
        for (int r = threadIdx.x; r < c.rows; r += kThreads)
            s_tok[r] = c.shared ? (c.m0 + r) : min(max(perm[c.hbase + c.m0 + r], 0), T * k - 1) / k;
        const int nbase = nt * BN + wave * 16 * NBW;

        f32x4 acc[kMB][2][NBW];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) acc[mb][m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kc = 0; kc < H; kc += kKC) {
            __syncthreads();               // previous chunk consumed; s_tok visible
            stage_a(s_a, c.rows, [&](int r) { return x + (size_t)s_tok[r] * H + kc; });
            u32x4 codes[2][NBW];
            float sc[2][NBW], bi[2][NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int n = nbase + nb * 16 + (lane & 15);
                load_b(Wset.gate, c.e, I, H, n, kc, lane, codes[0][nb], sc[0][nb], bi[0][nb]);
                load_b(Wset.up, c.e, I, H, n, kc, lane, codes[1][nb], sc[1][nb], bi[1][nb]);
            }
            __syncthreads();
            mma_chunk<2, NBW>(s_a, c.rows, lane, codes, sc, bi, acc);
        }
        // epilogue: h = silu(gate) * up
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
            if (mb * 16 >= c.rows) break;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int n = nbase + nb * 16 + (lane & 15);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = mb * 16 + (lane >> 4) * 4 + q;
                    if (m < c.rows) {
                        const float g = acc[mb][0][nb][q], u = acc[mb][1][nb][q];
                        h[(size_t)(c.hbase + c.m0 + m) * I + n] = (uint16_t)f32_to_bf16(silu(g) * u);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down + routing-weighted scatter-add
// ---------------------------------------------------------------------------
template <int NBW>
__global__ __launch_bounds__(kThreads, 2) void k_grouped_down(
    int T, int H, int I, int E, int k, W4Set routed, W4Set shared, int has_shared,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const uint16_t* __restrict__ h, float* __restrict__ accum) {
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kBM * kAStride];
    __shared__ int s_pre[kMaxSeg + 1];
    __shared__ int s_tmp[kThreads];
    __shared__ int s_tok[kBM];
    __shared__ float s_w[kBM];

    const int nseg = E + (has_shared ? 1 : 0);
    const int n_mt = build_mtile_prefix(offsets, E, T, k, has_shared, s_pre, s_tmp);
    constexpr int BN = 4 * 16 * NBW;
    const int NT = H / BN;
    const int total = ((n_mt + 7) / 8) * 8 * NT;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    for (int i = blockIdx.x; i < total; i += gridDim.x) {
        int mt, nt;
        tile_coords(i, NT, mt, nt);
        if (mt >= n_mt) continue;
        const TileCtx c = locate(mt, s_pre, nseg, E, T, k, offsets);
        const W4Set& Wset = c.shared ? shared : routed;
        __syncthreads();
        for (int r = threadIdx.x; r < c.rows; r += kThreads) {
            if (c.shared) { s_tok[r] = c.m0 + r; s_w[r] = 1.0f; }
            else {
                const int f = min(max(perm[c.hbase + c.m0 + r], 0), T * k - 1);
                s_tok[r] = f / k;
                s_w[r] = topk_w[f];
            }
        }
        const int nbase = nt * BN + wave * 16 * NBW;
        const uint16_t* hrow0 = h + (size_t)(c.hbase + c.m0) * I;

        f32x4 acc[kMB][1][NBW];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc[mb][0][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kc = 0; kc < I; kc += kKC) {
            __syncthreads();
            stage_a(s_a, c.rows, [&](int r) { return hrow0 + (size_t)r * I + kc; });
            u32x4 codes[1][NBW];
            float sc[1][NBW], bi[1][NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int n = nbase + nb * 16 + (lane & 15);
                load_b(Wset.down, c.e, H, I, n, kc, lane, codes[0][nb], sc[0][nb], bi[0][nb]);
            }
            __syncthreads();
            mma_chunk<1, NBW>(s_a, c.rows, lane, codes, sc, bi, acc);
        }
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
            if (mb * 16 >= c.rows) break;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int n = nbase + nb * 16 + (lane & 15);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = mb * 16 + (lane >> 4) * 4 + q;
                    if (m < c.rows)
                        unsafeAtomicAdd(accum + (size_t)s_tok[m] * H + n, s_w[m] * acc[mb][0][nb][q]);
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ acc,
                                                  uint16_t* __restrict__ out, long n) {
    for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (long)gridDim.x * 256 * 8) {
        const float4 a = *reinterpret_cast<const float4*>(acc + i);
        const float4 b = *reinterpret_cast<const float4*>(acc + i + 4);
        u32x4 o = {pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                   pack_bf16x2(b.z, b.w)};
        *reinterpret_cast<u32x4*>(out + i) = o;
    }
}

static int cu_count() {
    static int cached = 0;
    if (!cached) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cached = n;
        else
            cached = 256;
    }
    return cached;
}

hipError_t launch_forward_grouped(const ForwardArgs& a, hipStream_t st, KernelTimer& tm) {
    constexpr int NBW_GU = 2, NBW_DN = 2;
    const int nseg = a.E + (a.has_shared ? 1 : 0);
    // upper bound of M-tiles: every routed row tile-padded, plus one partial per segment
    const long mt_bound = ((long)a.T * a.k) / kBM + nseg + (a.has_shared ? a.T / kBM + 1 : 0);
    const int slots = cu_count() * 2;
    const long gu_tiles = mt_bound * (a.I / (64 * NBW_GU)) + 8;
    const long dn_tiles = mt_bound * (a.H / (64 * NBW_DN)) + 8;
    const int g_gu = (int)(((gu_tiles < slots ? gu_tiles : slots) + 7) / 8 * 8);
    const int g_dn = (int)(((dn_tiles < slots ? dn_tiles : slots) + 7) / 8 * 8);
    const long acc_elems = (long)a.T * a.H;

    tm.before();
    hipLaunchKernelGGL(k_grouped_gateup<NBW_GU>, dim3(g_gu), dim3(kThreads), 0, st, a.x, a.T,
                       a.H, a.I, a.E, a.k, a.routed, a.shared, a.has_shared, a.offsets, a.perm,
                       a.ws_h, a.ws_acc, acc_elems);
    tm.after();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    hipLaunchKernelGGL(k_grouped_down<NBW_DN>, dim3(g_dn), dim3(kThreads), 0, st, a.T, a.H, a.I,
                       a.E, a.k, a.routed, a.shared, a.has_shared, a.topk_w, a.offsets, a.perm,
                       a.ws_h, a.ws_acc);
    tm.after();
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const long nblk = (acc_elems / 8 + 255) / 256;
    tm.before();
    hipLaunchKernelGGL(k_finalize, dim3((unsigned)(nblk < 2048 ? nblk : 2048)), dim3(256), 0, st,
                       a.ws_acc, a.out, acc_elems);
    tm.after();
    return hipGetLastError();
}

}  // namespace moe_w4
