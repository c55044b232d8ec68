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
constexpr int kMaxSeg = 1025;
constexpr int kWaves = 8;                // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;

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

// ---------------------------------------------------------------------------
// The K-loop of one tile, software-pipelined:
//   A (kBM rows x kKC bf16 per chunk) is copied global -> LDS by the direct
//   global_load_lds_dwordx4 path (no registers), double buffered, one barrier
//   per chunk.  Each lane supplies its own source address, so the rows are
//   gathered by token on the fly and the 16-byte chunks of a row are stored
//   XOR-swizzled by row, which keeps the MFMA operand reads conflict-free.
//   B (codes, 128 bits per lane per 16-row block, plus the group's scale and
//   bias) goes straight to registers and is dequantised there.  The next
//   chunk's A and B are in flight while the current chunk's MFMAs run.
// ---------------------------------------------------------------------------
constexpr int kARow = kKC * 2;               // bytes of one A row per chunk (256)
constexpr int kABuf = kBM * kARow;           // bytes of one A buffer (32 KiB)
constexpr int kStages = 4;                   // K-loop pipeline depth
constexpr int kRowsPerWaveDma = kBM / kWaves;   // A rows copied by each wavefront
constexpr int kDmaPerWave = kRowsPerWaveDma / 4;  // 4 rows (1 KiB) per DMA instruction

template <int NMAT, int NBW>
struct BRegs {
    u32x4 c[NMAT][NBW];
    uint32_t s[NMAT][NBW];      // bf16 scale bits (combined only at use, so that
    uint32_t b[NMAT][NBW];      // issuing the loads never waits for them)
};

// Per-lane B addressing: element offsets of the lane's row within its matrix set.
template <int NMAT, int NBW>
struct BAddr {
    const uint8_t* codes[NMAT];      // matrix base (wave-uniform)
    const uint16_t* scales[NMAT];
    const uint16_t* biases[NMAT];
    uint32_t row[NBW];               // row index (expert * N + n) of each 16-row block
    int K;
    int lane;
};

// Loads of chunk kc; a dummy chunk (past the end of K) loads the first bytes of
// each matrix in every lane, one cache line per instruction, so that the number
// of loads per chunk never varies.
template <int NMAT, int NBW>
__device__ __forceinline__ void load_b_chunk(BRegs<NMAT, NBW>& r, const BAddr<NMAT, NBW>& a, int kc,
                                             bool dummy) {
    const int kq = a.K / kGroup;
    const int g = kc / kGroup + ((a.lane >> 4) >> 1);         // lanes 32..63 use the odd group
    const int cb = (kc >> 1) + (a.lane >> 4) * 16;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const size_t row = a.row[nb];
            const size_t co = dummy ? 0 : row * (size_t)(a.K / 2) + cb;
            const size_t so = dummy ? 0 : row * kq + g;
            r.c[m][nb] = load_u32x4(a.codes[m] + co);
            r.s[m][nb] = a.scales[m][so];
            r.b[m][nb] = a.biases[m][so];
        }
}

// 16 bytes per lane, global -> LDS, written at lds + 16 * lane (lds is the same for
// the whole wavefront).  Issued through inline assembly so that the compiler's
// wait insertion does not see it: it would otherwise wait for every in-flight
// copy at each barrier, which serialises the pipeline.  The K-loop waits for the
// copies explicitly with vmcnt; M0 is restored after use.
__device__ __forceinline__ void dma16_to_lds(const void* src, void* lds) {
    const uint32_t l = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(l)
        : "memory");
}

// A rows of a tile: row r starts at base + rowidx(r) * row_bytes, where rowidx is
// the token (gathered rows) or the consecutive h row.
struct ASrc {
    const uint8_t* base;
    size_t row_bytes;
    int rowidx[kDmaPerWave];   // row index of the lane's row in each DMA instruction
};

// Issue the DMA of one A chunk: wavefront w copies rows [16w, 16w+16), four rows
// (64 lanes x 16 bytes) per instruction.  Rows past the tile's valid rows re-read
// its last valid row, so every address stays inside the operand.
__device__ __forceinline__ void issue_a_dma(uint8_t* s_buf, int wave, int lane, const ASrc& a,
                                            int kc_bytes, bool dummy) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int r0 = wave * kRowsPerWaveDma + i * 4;
        const int lrow = r0 + (lane >> 4);
        const int logical = (lane & 15) ^ (lrow & 15);
        const uint8_t* src = dummy ? a.base
                                   : a.base + (size_t)a.rowidx[i] * a.row_bytes + kc_bytes + logical * 16;
        dma16_to_lds(src, s_buf + r0 * kARow);
    }
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// One K chunk of MFMAs over MB valid 16-row blocks (compile-time, so each step
// is branch-free and the A-fragment reads of a step are issued together).
template <int NMAT, int NBW, int MB>
__device__ __forceinline__ void mma_chunk(const uint8_t* s_a, int lane, const BRegs<NMAT, NBW>& br,
                                          f32x4 (&acc)[MB][NMAT][NBW]) {
    const int arow = lane & 15;
    const int agrp = (lane >> 4) * 4;      // logical 16-byte chunk of the lane's 32 k values
    const uint32_t magic = 0x64006400u;
    DqConst q[NMAT][NBW];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            q[m][nb] = make_dq(bf16_to_f32(br.s[m][nb]), bf16_to_f32(br.b[m][nb]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = ((agrp + j) ^ arow) * 16;
        bf16x8 a[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            a[mb] = *reinterpret_cast<const bf16x8*>(s_a + (mb * 16 + arow) * kARow + col);
        bf16x8 b[NMAT][NBW];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const uint32_t d = (j == 0) ? br.c[m][nb].x : (j == 1) ? br.c[m][nb].y
                                 : (j == 2) ? br.c[m][nb].z : br.c[m][nb].w;
                b[m][nb] = dequant8_mix(d, q[m][nb], magic);
            }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    acc[mb][m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b[m][nb],
                                                                            acc[mb][m][nb], 0, 0, 0);
    }
}

// Issue the loads of one K chunk: the A DMA first, then B to registers.  The
// order matters for the vmcnt accounting in tile_kloop.
template <int NMAT, int NBW>
__device__ __forceinline__ void issue_chunk(BRegs<NMAT, NBW>& br, const BAddr<NMAT, NBW>& ba,
                                            uint8_t* s_stage, int wave, int lane, const ASrc& src,
                                            int kc, bool dummy) {
    issue_a_dma(s_stage, wave, lane, src, 2 * kc, dummy);
    load_b_chunk(br, ba, kc, dummy);
}

// Vector-memory instructions one issue_chunk emits per wavefront.
template <int NMAT, int NBW>
constexpr int kLoadsPerChunk = kDmaPerWave + 3 * NMAT * NBW;

// K-loop with a D-stage ring: chunk c lives in LDS stage c % D and register set
// c % D; chunks c+1 .. c+D-2 are in flight while chunk c is multiplied.  Every
// iteration issues exactly one chunk (a dummy one past the end of K), so the
// number of loads queued behind chunk c is always the same: its own B loads and
// D-2 whole chunks.  Loads complete in order, so waiting until at most that many
// are outstanding means chunk c has landed.
template <int NMAT, int NBW, int D, int MB>
__device__ __forceinline__ void tile_kloop(uint8_t* s_a, int K, int wave, int lane,
                                           const ASrc& src, const BAddr<NMAT, NBW>& ba,
                                           f32x4 (&acc)[MB][NMAT][NBW]) {
    static_assert(D >= 2 && D <= 4, "pipeline depth");
    constexpr int kBehind = 3 * NMAT * NBW + (D - 2) * kLoadsPerChunk<NMAT, NBW>;
    static_assert(kBehind < 64, "pipeline too deep for vmcnt");
    const int nch = K / kKC;
    BRegs<NMAT, NBW> br[D];
#pragma unroll
    for (int st = 0; st < D - 1; ++st)
        issue_chunk(br[st], ba, s_a + st * kABuf, wave, lane, src, st * kKC, st >= nch);
    const int nit = (nch + D - 1) / D * D;
    for (int base = 0; base < nit; base += D) {
#pragma unroll
        for (int st = 0; st < D; ++st) {
            const int c = base + st;
            wait_vmcnt<kBehind>();
            __syncthreads();       // chunk c visible to all; chunk c-1's stage is free
            const int nxt = (st + D - 1) % D;
            issue_chunk(br[nxt], ba, s_a + nxt * kABuf, wave, lane, src, (c + D - 1) * kKC,
                        c + D - 1 >= nch);
            if (c < nch) mma_chunk<NMAT, NBW, MB>(s_a + st * kABuf, lane, br[st], acc);
        }
    }
    wait_vmcnt<0>();               // drain the dummy loads
    __syncthreads();               // all stages free for the next tile
}

// ---------------------------------------------------------------------------
// Per-tile bodies, specialised on the number MB of valid 16-row blocks
// ---------------------------------------------------------------------------
template <int NBW, int MB>
__device__ __forceinline__ void gateup_tile(uint8_t* s_a, int H, int I, int wave, int lane,
                                            const ASrc& src, const BAddr<2, NBW>& ba, int rows,
                                            int rowbase, int nbase, uint16_t* __restrict__ h) {
    f32x4 acc[MB][2][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc[mb][m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile_kloop<2, NBW, kStages, MB>(s_a, H, wave, lane, src, ba, acc);
    // epilogue: h = silu(gate) * up, bf16, expert-sorted rows
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int n = nbase + nb * 16 + (lane & 15);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = mb * 16 + (lane >> 4) * 4 + q;
                if (m < rows) {
                    const float g = acc[mb][0][nb][q], u = acc[mb][1][nb][q];
                    h[(size_t)(rowbase + m) * I + n] = (uint16_t)f32_to_bf16(silu(g) * u);
                }
            }
        }
}

template <int NBW, int MB>
__device__ __forceinline__ void down_tile(uint8_t* s_a, int H, int I, int wave, int lane,
                                          const ASrc& src, const BAddr<1, NBW>& ba, int rows,
                                          int nbase, const int* s_tok, const float* s_w,
                                          float* __restrict__ accum) {
    f32x4 acc[MB][1][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[mb][0][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile_kloop<1, NBW, kStages, MB>(s_a, I, wave, lane, src, ba, acc);
    // epilogue: routing-weighted add into the token's fp32 accumulator row
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int n = nbase + nb * 16 + (lane & 15);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = mb * 16 + (lane >> 4) * 4 + q;
                if (m < rows) unsafeAtomicAdd(accum + (size_t)s_tok[m] * H + n, s_w[m] * acc[mb][0][nb][q]);
            }
        }
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
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kStages * kABuf];
    __shared__ int s_pre[kMaxSeg + 1];
    __shared__ int s_tmp[kThreads];
    __shared__ int s_tok[kBM];

    // clear the fp32 output accumulator for the down kernel
    for (long i = ((long)blockIdx.x * kThreads + threadIdx.x) * 4; i < acc_elems;
         i += (long)gridDim.x * kThreads * 4)
        *reinterpret_cast<float4*>(acc_zero + i) = float4{0.f, 0.f, 0.f, 0.f};

    const int nseg = E + (has_shared ? 1 : 0);
    const int n_mt = build_mtile_prefix(offsets, E, T, k, has_shared, s_pre, s_tmp);
    constexpr int BN = kWaves * 16 * NBW;
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
        __syncthreads();                 // previous tile's readers are done
        for (int r = threadIdx.x; r < c.rows; r += kThreads)
            s_tok[r] = c.shared ? (c.m0 + r) : min(max(perm[c.hbase + c.m0 + r], 0), T * k - 1) / k;
        __syncthreads();
        const int nbase = nt * BN + wave * 16 * NBW;

        BAddr<2, NBW> ba;
        ba.codes[0] = Wset.gate.codes; ba.scales[0] = Wset.gate.scales; ba.biases[0] = Wset.gate.biases;
        ba.codes[1] = Wset.up.codes;   ba.scales[1] = Wset.up.scales;   ba.biases[1] = Wset.up.biases;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) ba.row[nb] = (uint32_t)(c.e * I + nbase + nb * 16 + (lane & 15));
        ba.K = H;
        ba.lane = lane;
        ASrc src;
        src.base = reinterpret_cast<const uint8_t*>(x);
        src.row_bytes = (size_t)H * 2;
#pragma unroll
        for (int q = 0; q < kDmaPerWave; ++q)
            src.rowidx[q] = s_tok[min(wave * kRowsPerWaveDma + q * 4 + (lane >> 4), c.rows - 1)];

        const int rowbase = c.hbase + c.m0;
        switch ((c.rows + 15) >> 4) {
            case 1: gateup_tile<NBW, 1>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
            case 2: gateup_tile<NBW, 2>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
            case 3: gateup_tile<NBW, 3>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
            case 4: gateup_tile<NBW, 4>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
            case 5: gateup_tile<NBW, 5>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
            case 6: gateup_tile<NBW, 6>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
            case 7: gateup_tile<NBW, 7>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
            default: gateup_tile<NBW, 8>(s_a, H, I, wave, lane, src, ba, c.rows, rowbase, nbase, h); break;
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
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kStages * kABuf];
    __shared__ int s_pre[kMaxSeg + 1];
    __shared__ int s_tmp[kThreads];
    __shared__ int s_tok[kBM];
    __shared__ float s_w[kBM];

    const int nseg = E + (has_shared ? 1 : 0);
    const int n_mt = build_mtile_prefix(offsets, E, T, k, has_shared, s_pre, s_tmp);
    constexpr int BN = kWaves * 16 * NBW;
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
        BAddr<1, NBW> ba;
        ba.codes[0] = Wset.down.codes; ba.scales[0] = Wset.down.scales; ba.biases[0] = Wset.down.biases;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) ba.row[nb] = (uint32_t)(c.e * H + nbase + nb * 16 + (lane & 15));
        ba.K = I;
        ba.lane = lane;
        ASrc src;
        src.base = reinterpret_cast<const uint8_t*>(h + (size_t)(c.hbase + c.m0) * I);
        src.row_bytes = (size_t)I * 2;
#pragma unroll
        for (int q = 0; q < kDmaPerWave; ++q)
            src.rowidx[q] = min(wave * kRowsPerWaveDma + q * 4 + (lane >> 4), c.rows - 1);

        switch ((c.rows + 15) >> 4) {
            case 1: down_tile<NBW, 1>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
            case 2: down_tile<NBW, 2>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
            case 3: down_tile<NBW, 3>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
            case 4: down_tile<NBW, 4>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
            case 5: down_tile<NBW, 5>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
            case 6: down_tile<NBW, 6>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
            case 7: down_tile<NBW, 7>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
            default: down_tile<NBW, 8>(s_a, H, I, wave, lane, src, ba, c.rows, nbase, s_tok, s_w, accum); break;
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
    constexpr int NBW_GU = 1, NBW_DN = 2;
    const int nseg = a.E + (a.has_shared ? 1 : 0);
    // upper bound of M-tiles: every routed row tile-padded, plus one partial per segment
    const long mt_bound = ((long)a.T * a.k) / kBM + nseg + (a.has_shared ? a.T / kBM + 1 : 0);
    const int slots = cu_count();          // one 8-wave workgroup per CU
    const long gu_tiles = mt_bound * (a.I / (kWaves * 16 * NBW_GU)) + 8;
    const long dn_tiles = mt_bound * (a.H / (kWaves * 16 * NBW_DN)) + 8;
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
