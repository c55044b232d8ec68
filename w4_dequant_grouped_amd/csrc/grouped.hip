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
//   k_grouped_gateup  per tile (segment, 64-row M-tile, 64-column N-tile of I):
//                     the rows' activations (gathered by token), the gate and up
//                     codes and their scale/bias words are copied into LDS; each
//                     wavefront dequantises its 16 weight rows (w = c * s + b,
//                     fp32, RNE to bf16) into the MFMA B operand and multiplies on
//                     v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the
//                     epilogue applies SwiGLU and writes h (bf16) in expert-sorted
//                     row order.
//   k_grouped_down    same K-loop over h (rows contiguous per expert); the epilogue
//                     scales each row by its routing weight and stores it (bf16) as
//                     row t*k + j of a per-(token, slot) buffer, the shared expert's
//                     row of token t as row T*k + t.  Plain stores: no atomics, and
//                     every output row is owned by exactly one tile row.
//   k_finalize        out[t] = sum of token t's k slot rows and its shared row, in
//                     slot order, in fp32, rounded to bf16 (deterministic).
// A segment is a routed expert's rows (offsets[e]..offsets[e+1], tokens via the
// permutation) or the shared expert's rows (all tokens, weight 1).  Persistent
// 4-wavefront workgroups, three per CU, take tiles from per-XCD queues; each
// queue is a contiguous run of the tile sequence, in which blocks of up to four
// M-tiles of one segment take each N-tile together, so a weight tile is fetched
// into an XCD's L2 once per block rather than once per M-tile.
//
// MFMA operand layout used (16x16x32, wave64): lane l supplies A row l%16 and B
// column l%16, each with 8 k values for the k-slot group l/16; D element
// (4*(l/16)+i, l%16) is accumulator i of lane l.  A lane holds 32 consecutive
// codes of one weight row (k = 32*(l/16) .. +32 of a 128-wide K chunk); MFMA step
// j consumes its 8 codes 8j..8j+7, and the A operand is read from LDS at the same
// logical k, so both operands agree on the k order.
#include "device.h"
#include "kernels.h"
#include "lds_copy.h"

namespace moe_w4 {

constexpr int kBM = 64;                // rows per M-tile
constexpr int kMB = kBM / 16;          // 16-row MFMA blocks per M-tile
static_assert(kMB == 4, "the per-tile dispatch below covers 1..4 row blocks");
constexpr int kKC = 128;               // K per chunk (4 MFMA steps of 32)
constexpr int kWaves = 4;                // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kWgPerCu = 3;              // resident workgroups per CU (persistent grid size)

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
// Segment at sequence position p: the shared expert first (when present), then
// the routed experts in id order.
__device__ __forceinline__ int seq_segment(int p, int E, int has_shared) {
    return has_shared ? (p == 0 ? E : p - 1) : p;
}

__device__ int build_mtile_prefix(const int32_t* __restrict__ offsets, int E, int T, int k,
                                  int has_shared, int* s_pre, int* s_tmp) {
    const int nseg = E + (has_shared ? 1 : 0);
    const int tid = threadIdx.x;
    // each thread sums a contiguous run of segments
    const int per = (nseg + kThreads - 1) / kThreads;
    const int s0 = min(tid * per, nseg), s1 = min(s0 + per, nseg);
    int local = 0;
    for (int s = s0; s < s1; ++s) local += (seg_count(offsets, seq_segment(s, E, has_shared), E, T, k) + kBM - 1) / kBM;
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
        run += (seg_count(offsets, seq_segment(s, E, has_shared), E, T, k) + kBM - 1) / kBM;
    }
    if (tid == kThreads - 1) s_pre[nseg] = s_tmp[kThreads - 1];
    __syncthreads();
    return s_pre[nseg];
}

// Last sequence position s with s_pre[s] <= key.  s_pre is nondecreasing and
// s_pre[0] = 0, so that is the number of positions with s_pre[s] <= key, minus
// one: the lanes test 64 positions per step with one LDS read each, and the
// reads of all steps are independent (one LDS round trip instead of a chain).
__device__ __forceinline__ int find_segment(const int* s_pre, int nseg, int key, int lane) {
    int cnt = 0;
    for (int base = 0; base < nseg; base += kWave) {
        const int s = base + lane;
        const bool ok = (s < nseg) && (s_pre[min(s, nseg - 1)] <= key);
        cnt += __popcll(__ballot(ok));
    }
    return (int)__builtin_amdgcn_readfirstlane(cnt - 1);
}

__device__ __forceinline__ TileCtx locate(int pos, int mt, const int* s_pre, int E, int T, int k,
                                          int has_shared, const int32_t* __restrict__ offsets) {
    // every lane holds the same values: keep them in scalar registers
    TileCtx c;
    const int seg = seq_segment(pos, E, has_shared);
    c.seg = seg;
    c.shared = (seg >= E);
    c.e = c.shared ? 0 : seg;
    c.m0 = (int)__builtin_amdgcn_readfirstlane((mt - s_pre[pos]) * kBM);
    c.rows = (int)__builtin_amdgcn_readfirstlane(min(kBM, seg_count(offsets, seg, E, T, k) - c.m0));
    c.hbase = (int)__builtin_amdgcn_readfirstlane(seg_first(offsets, seg, E, T, k));
    return c;
}

// Tile order.  The n_mt * NT tiles form one sequence: segment by segment (the
// shared expert, whose M-tiles are all full, first, so that the list does not
// end on them), each segment's M-tiles in blocks of kMtBlock, and within a block
// N-tile by N-tile, the block's M-tiles innermost.  The tiles of one block that share an N-tile
// read the same weight tile, and the NT tiles of one M-tile read the same
// gathered activation rows; consecutive entries are taken at nearly the same
// time by the workgroups of one XCD, so both kinds of operand reach that XCD's
// L2 once instead of once per M-tile (weights) or per N-tile (activations).
constexpr int kMtBlock = 4;

// q / d for 0 <= q and d = 1..4 (the M-tiles of a block), by constant divisors.
__device__ __forceinline__ int div_small(int q, int d) {
    return d == 4 ? (q >> 2) : d == 3 ? q / 3 : d == 2 ? (q >> 1) : q;
}

// Sequence entry e -> (sequence position of its segment, global M-tile index,
// N-tile).  s_pre is the exclusive M-tile prefix over the segments in sequence
// order (seq_segment gives the segment at a position); position s holds entries
// [s_pre[s] * NT, s_pre[s + 1] * NT).
__device__ __forceinline__ void tile_coords(int e, int NT, const int* s_pre, int nseg, int lane,
                                            int& pos, int& mt, int& nt) {
    static_assert(kMtBlock >= 1 && kMtBlock <= 4, "div_small covers blocks of up to 4 M-tiles");
    pos = find_segment(s_pre, nseg, e / NT, lane);   // s_pre[s] * NT <= e  <=>  s_pre[s] <= e / NT
    const int first = s_pre[pos];
    const int m_s = s_pre[pos + 1] - first;
    const int r = e - first * NT;
    const int b = r / (kMtBlock * NT);
    const int rr = r - b * (kMtBlock * NT);
    const int cnt = min(kMtBlock, m_s - b * kMtBlock);
    nt = div_small(rr, cnt);
    mt = first + b * kMtBlock + (rr - nt * cnt);
}

// The sequence is cut into 8 contiguous queues of nearly equal length in the
// control block.  Workgroup b runs on XCD b mod 8 (round-robin dispatch) and
// serves queue b mod 8 first, so each queue's blocks are normally processed by
// the workgroups of one XCD.  A workgroup whose queue is empty takes tiles from
// the others.
__device__ __forceinline__ int queue_start(int q, int n_mt, int NT) {
    return (int)(((long long)n_mt * NT * q) >> 3);
}
__device__ __forceinline__ int queue_len(int q, int n_mt, int NT) {
    return queue_start(q + 1, n_mt, NT) - queue_start(q, n_mt, NT);
}

// `qb` is the first queue word of a kernel's set in the control block.
__device__ __forceinline__ uint32_t queue_take(uint32_t* qb, int q) {
    return __hip_atomic_fetch_add(qb + q * kCtlQueueStride, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

// Next tile index for this workgroup, or -1 when every queue is empty.  `q`
// is the queue to try first and, on success, the queue the tile came from;
// `empty` remembers the queues already found empty.
__device__ __forceinline__ int grab_tile(uint32_t* qb, int n_mt, int NT, int& q, uint32_t& empty) {
    for (int d = 0; d < 8; ++d) {
        const int qq = (q + d) & 7;
        if (empty & (1u << qq)) continue;
        const int lim = queue_len(qq, n_mt, NT);
        if (lim > 0) {
            const uint32_t j = queue_take(qb, qq);
            if (j < (uint32_t)lim) {           // unsigned: any stale value past the queue is empty
                q = qq;
                return queue_start(qq, n_mt, NT) + (int)j;
            }
        }
        empty |= 1u << qq;
    }
    return -1;
}

// Tile scheduling state of a workgroup (meaningful in thread 0 only).  A tile
// is taken only once the workgroup is free to run it: an entry taken while the
// previous tile still runs would be held back for a whole tile time, and near
// the end of the list other workgroups would find the queues empty and leave
// while such entries wait.  `ran` counts the tiles the workgroup ran.
struct TileQueue {
    int q;               // current queue
    uint32_t empty;      // queues found empty
    uint32_t ran;
    __device__ __forceinline__ int next(uint32_t* qb, int n_mt, int NT) {
        return grab_tile(qb, n_mt, NT, q, empty);
    }
};

// Exit accounting of a grouped GEMM: one 64-bit word holds the workgroups that
// have left (high half) and the tiles they ran (low half), updated with one
// atomic per workgroup.  In a call that found its queue words zero, arrival
// counts stay below the grid size and the last workgroup out sees every tile of
// the list run; anything else means the control block was dirty (not
// zero-filled, or shared with a concurrent call), which is counted in the error
// word.  The queues and this word are cleared by k_finalize, the call's last
// kernel, so the next call starts clean either way.
__device__ __forceinline__ void report_exit(uint32_t* ctl, int exit_word, uint32_t ran, uint32_t tiles) {
    if (threadIdx.x == 0) {
        uint64_t* w = reinterpret_cast<uint64_t*>(ctl + exit_word);
        const uint64_t prev = __hip_atomic_fetch_add(w, (1ull << 32) | ran, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t arrived = (uint32_t)(prev >> 32);
        const bool dirty = arrived >= gridDim.x ||
                           (arrived == gridDim.x - 1 && (uint32_t)prev + ran != tiles);
        if (dirty) __hip_atomic_fetch_add(ctl + kCtlErrors, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// The K-loop of one tile, software-pipelined through LDS.
//   The operand bytes of a K chunk -- the kBM activation rows (A) and the
//   wavefront's packed weight rows (B codes) -- are copied global -> LDS by the
//   direct global_load_lds path, issued through inline assembly, into one of two
//   stages: while chunk c is multiplied from one stage, chunk c+1 is copied into
//   the other.  The copies' only waits are explicit.  A rows are gathered by
//   token on the fly and stored XOR-swizzled by row, which keeps the MFMA operand
//   reads conflict-free.  The group scale/bias words travel in registers instead:
//   each lane loads the words of its (array, row) for four chunks with one
//   16-byte load and hands each chunk's word to the lanes that need it with
//   ds_bpermute.  (Copied to LDS one word per lane and chunk, as before, those
//   loads were a quarter of a chunk's copy instructions and most of its memory
//   requests, 64 scattered 4-byte reads; a timing copy without them was 14%
//   faster on gate/up at 512 tokens.)
// ---------------------------------------------------------------------------
constexpr int kARow = kKC * 2;                     // bytes of one A row per chunk (256)
constexpr int kABuf = kBM * kARow;                 // A bytes per stage (16 KiB)
constexpr int kBRowBytes = kKC / 2;                // packed codes of a weight row per chunk (64)
constexpr int kBBlk = 16 * kBRowBytes;             // codes of one 16-row block (1 KiB)
constexpr int kBlkPerWave = 2;                     // (matrix, 16-row block) pairs per wavefront
constexpr int kBBuf = kWaves * kBlkPerWave * kBBlk;    // B code bytes per stage (8 KiB)
constexpr int kStageBytes = kABuf + kBBuf;
constexpr int kStages = 2;                         // 48 KiB: three workgroups share a CU's 160 KiB
constexpr int kDmaPerWave = kBM / kWaves / 4;      // A copies per wavefront in a full tile (4 rows, 1 KiB each)

// Per-tile copy addressing.  The bases are wave-uniform (SGPRs, advanced per
// chunk with scalar adds); the lane offsets are computed once per tile, so a
// copy costs no vector arithmetic.
template <int NMAT, int NBW>
struct TileSrc {
    uint64_t a_base;                 // A operand (x for gate/up, the segment's h rows for down)
    uint32_t a_off[kDmaPerWave];     // lane's byte offset of its row piece in each A copy
    uint64_t b_base[NMAT][NBW];      // codes of the first row of each (matrix, 16-row block)
    uint32_t b_off;                  // lane's byte offset within a block's chunk
    uint64_t sb_addr;                // the scale/bias words of the lane's (array, row), chunk 0 first
    int K;
};

// Offsets of a stage's parts from the start of the stage ring.
__device__ __forceinline__ uint32_t off_a(int st) { return (uint32_t)(st * kStageBytes); }
__device__ __forceinline__ uint32_t off_b(int st, int wave) {
    return (uint32_t)(st * kStageBytes + kABuf + wave * kBlkPerWave * kBBlk);
}

// Lane offsets of the A copies: copy i of wavefront w moves the four rows of
// group g = w + 4 i (rows 4 g .. 4 g + 3; 64 lanes x 16 bytes), so a tile of MB
// row blocks takes exactly MB copies from every wavefront and no wavefront
// waits longer than the others at the chunk barrier.  The lane's row is lrow and
// its 16-byte piece is stored XOR-swizzled by row.  row_of(lrow) gives the source
// row index (clamped by the caller to the tile's rows, so every address stays
// inside the operand).
template <typename RowOf>
__device__ __forceinline__ void a_offsets(uint32_t (&off)[kDmaPerWave], int wave, int lane,
                                          uint32_t row_bytes, RowOf row_of) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int lrow = (wave + kWaves * i) * 4 + (lane >> 4);
        const int logical = (lane & 15) ^ (lrow & 15);
        off[i] = (uint32_t)row_of(lrow) * row_bytes + (uint32_t)logical * 16u;
    }
}

// B addressing of a tile:
//  * codes: one copy per (matrix, 16-row block) pair p; lane L fills slot L&3
//    (16 bytes) of row r = L>>2 (64 B per row) with quarter (L&3) ^ ((r>>2)&3)
//    of the row's 64 code bytes of the chunk; the XOR spreads the 16 rows'
//    reads of one quarter over the LDS banks;
//  * scale/bias: lane L owns row L&15 of pair p = L>>5, in the scales (bit 4 of
//    L clear) or the biases; the row's word of chunk c holds the chunk's two
//    groups (even group in the low half) at sb_addr + 4 c.  Every word is 4-byte
//    aligned because K/64 is even and the arrays are 4-byte aligned.
template <int NMAT, int NBW>
__device__ __forceinline__ void b_addressing(TileSrc<NMAT, NBW>& t, const W4 (&mat)[NMAT],
                                             const uint32_t (&rowblk)[NBW], int K, int lane) {
    static_assert(NMAT * NBW == kBlkPerWave, "B slice layout");
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            t.b_base[m][nb] = uniform64((uint64_t)mat[m].codes + (uint64_t)rowblk[nb] * (uint64_t)(K / 2));
    t.b_off = (uint32_t)(lane >> 2) * (uint32_t)(K / 2) + (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
    // per-lane choice of array and row by bit masks on the wave-uniform values, so
    // that no array of a struct is indexed by a lane-varying value
    const uint64_t second = 0ull - (uint64_t)(lane >> 5);          // pair 1: all ones
    const uint64_t bias = 0ull - (uint64_t)((lane >> 4) & 1);       // biases: all ones
    const uint64_t sc0 = (uint64_t)mat[0].scales, sc1 = (uint64_t)mat[NMAT - 1].scales;
    const uint64_t bi0 = (uint64_t)mat[0].biases, bi1 = (uint64_t)mat[NMAT - 1].biases;
    const uint64_t m2 = (NMAT == 2) ? second : 0ull;
    const uint64_t sc = sc0 ^ ((sc0 ^ sc1) & m2), bi = bi0 ^ ((bi0 ^ bi1) & m2);
    const uint64_t arr = sc ^ ((sc ^ bi) & bias);
    const uint32_t r0 = rowblk[0], r1 = rowblk[NBW - 1];
    const uint32_t rb = r0 ^ ((r0 ^ r1) & ((NBW == 2) ? (uint32_t)second : 0u));
    t.sb_addr = arr + 2ull * ((uint64_t)(rb + (lane & 15)) * (uint64_t)(K / kGroup));
    t.K = K;
}

// Copies of chunk c into stage c mod kStages: the wavefront's MB A copies (row
// groups of the tile's row blocks only), then its B code blocks -- the same
// count for every wavefront.
template <int MB, int NMAT, int NBW>
__device__ __forceinline__ void issue_chunk(uint32_t ring, int wave, const TileSrc<NMAT, NBW>& t, int c) {
    const int st = c % kStages;
    {
        const uint64_t ab = t.a_base + (uint64_t)c * (kKC * 2);
#pragma unroll
        for (int i = 0; i < MB; ++i)
            dma16_to_lds(ab, t.a_off[i], ring + off_a(st) + (wave + kWaves * i) * 4 * kARow);
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            dma16_to_lds(t.b_base[m][nb] + (uint64_t)c * (kKC / 2), t.b_off,
                         ring + off_b(st, wave) + (m * NBW + nb) * kBBlk);
}

// The lane's scale/bias words of chunks 4 b .. 4 b + 3 (one 16-byte load, 4-byte
// aligned); for a last block of fewer chunks, dword loads that stay inside the
// row (the words past its last chunk are never used).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ u32x4 load_sb_block(uint64_t sb_addr, int b, int nch) {
    // a global (not flat) pointer: a flat load would also count against the LDS
    // wait counter
    const __attribute__((address_space(1))) uint32_t* p =
        reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(sb_addr) + 4 * b;
    if (4 * b + 4 <= nch) {
        const u32x4_a4 v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4_a4*>(p);
        return u32x4{v.x, v.y, v.z, v.w};
    }
    const int last = nch - 1 - 4 * b;
    return u32x4{p[0], p[min(1, last)], p[min(2, last)], p[min(3, last)]};
}


// Operands of one K chunk that are read before the chunk's MFMA work: the
// wavefront's packed codes and the A fragments of the first MFMA step from LDS,
// and the scale/bias words from the lanes that hold them.  They are read right after the barrier that publishes the
// chunk, ahead of the next chunk's copy instructions, so their LDS latency
// overlaps the copy issue instead of stalling the first dequantisation.
template <int NMAT, int NBW, int MB>
struct ChunkOps {
    u32x4 codes[NMAT][NBW];
    uint32_t sw[NMAT][NBW], bw[NMAT][NBW];
    bf16x8 a0[MB];
};

// A fragments of MFMA step j: row (mb * 16 + lane % 16), the lane's logical
// 16-byte piece (4 * (lane / 16) + j), stored XOR-swizzled by row.
template <int MB>
__device__ __forceinline__ void read_a_step(bf16x8 (&a)[MB], const uint8_t* s_a, int lane, int j) {
    const int arow = lane & 15;
    const int col = (((lane >> 4) * 4 + j) ^ arow) * 16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(s_a + (mb * 16 + arow) * kARow + col);
}

// `mine` is this lane's scale/bias word of the chunk; the scale and bias of row
// arow of pair p are the words of lanes 32 p + arow and 32 p + 16 + arow.
template <int NMAT, int NBW, int MB>
__device__ __forceinline__ void read_chunk_ops(ChunkOps<NMAT, NBW, MB>& o, const uint8_t* s_a,
                                               const uint8_t* s_b, uint32_t mine, int lane) {
    const int arow = lane & 15;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int p = m * NBW + nb;
            o.sw[m][nb] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (p * 32 + arow), (int)mine);
            o.bw[m][nb] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (p * 32 + 16 + arow), (int)mine);
            o.codes[m][nb] = *reinterpret_cast<const u32x4*>(
                s_b + p * kBBlk + arow * kBRowBytes + (((lane >> 4) ^ (arow >> 2)) & 3) * 16);
        }
    read_a_step<MB>(o.a0, s_a, lane, 0);
}

// One K chunk of MFMAs over MB valid 16-row blocks (compile-time, so each step
// is branch-free).  The A fragments of step j + 1 are read before step j's
// dequantisation and MFMAs (two register sets in turn); a scheduling barrier
// keeps the compiler from sinking those reads next to their use, where each
// pair of MFMAs would wait a full LDS round trip.
template <int NMAT, int NBW, int MB>
__device__ __forceinline__ void mma_chunk(ChunkOps<NMAT, NBW, MB>& o, const uint8_t* s_a, int lane,
                                          f32x4 (&acc)[MB][NMAT][NBW]) {
    const uint32_t magic = 0x64006400u;
    const int half = (lane >> 5) * 16;     // lanes 32..63 take the chunk's odd group
    DqConst q[NMAT][NBW];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            q[m][nb] = make_dq(bf16_to_f32((o.sw[m][nb] >> half) & 0xFFFFu),
                               bf16_to_f32((o.bw[m][nb] >> half) & 0xFFFFu));
    bf16x8 a1[MB];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bf16x8 (&cur)[MB] = (j & 1) ? a1 : o.a0;
        bf16x8 (&nxt)[MB] = (j & 1) ? o.a0 : a1;
        if (j < 3) read_a_step<MB>(nxt, s_a, lane, j + 1);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 b[NMAT][NBW];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const uint32_t d = (j == 0) ? o.codes[m][nb].x : (j == 1) ? o.codes[m][nb].y
                                 : (j == 2) ? o.codes[m][nb].z : o.codes[m][nb].w;
                b[m][nb] = dequant8_mix(d, q[m][nb], magic);
            }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    acc[mb][m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[mb], b[m][nb],
                                                                            acc[mb][m][nb], 0, 0, 0);
    }
}

// K-loop over the two-stage ring.  Iteration c waits for this wavefront's copies
// (vmcnt 0), then a barrier makes every wavefront's part of chunk c visible and
// frees the stage read in iteration c-1, which receives chunk c+1 while chunk c
// is multiplied.  The chunk's first operands are read before the copies of chunk
// c+1 are issued.  The loop is unrolled by two so that each stage's LDS offsets
// are compile-time constants.  Nothing is copied past the end of K.  sbc holds
// the lane's scale/bias words of the current block of four chunks; at the first
// chunk of a block it takes sbn, and the next block's load goes out (its result
// is waited for with the copies of the next iteration).
template <int NMAT, int NBW, int MB, int ST>
__device__ __forceinline__ void kloop_step(uint8_t* s_stage, uint32_t ring, int wave, int lane,
                                           const TileSrc<NMAT, NBW>& t, int c, int nch,
                                           u32x4& sbc, u32x4& sbn, f32x4 (&acc)[MB][NMAT][NBW]) {
    wait_vmcnt<0>();
    __syncthreads();           // chunk c visible to all; the other stage is free
    if (ST == 0 && (c & 3) == 0) {
        sbc = sbn;
        if (c + 4 < nch) sbn = load_sb_block(t.sb_addr, c / 4 + 1, nch);
    }
    // c & 1 == ST
    const uint32_t mine = (c & 2) ? sbc[ST + 2] : sbc[ST];
    ChunkOps<NMAT, NBW, MB> o;
    read_chunk_ops<NMAT, NBW, MB>(o, s_stage + off_a(ST), s_stage + off_b(ST, wave), mine, lane);
    if (c + 1 < nch) issue_chunk<MB>(ring, wave, t, c + 1);
    mma_chunk<NMAT, NBW, MB>(o, s_stage + off_a(ST), lane, acc);
}

template <int NMAT, int NBW, int MB>
__device__ __forceinline__ void tile_kloop(uint8_t* s_stage, int wave, int lane,
                                           const TileSrc<NMAT, NBW>& t,
                                           f32x4 (&acc)[MB][NMAT][NBW]) {
    static_assert(kStages == 2, "the loop below alternates two stages");
    const int nch = t.K / kKC;
    const uint32_t ring = lds_addr(s_stage);
    u32x4 sbc, sbn = load_sb_block(t.sb_addr, 0, nch);
    issue_chunk<MB>(ring, wave, t, 0);
    for (int c = 0; c < nch; c += 2) {
        kloop_step<NMAT, NBW, MB, 0>(s_stage, ring, wave, lane, t, c, nch, sbc, sbn, acc);
        if (c + 1 < nch) kloop_step<NMAT, NBW, MB, 1>(s_stage, ring, wave, lane, t, c + 1, nch, sbc, sbn, acc);
    }
    __syncthreads();           // both stages free for the next tile
}

// ---------------------------------------------------------------------------
// Per-tile bodies, specialised on the number MB of valid 16-row blocks
// ---------------------------------------------------------------------------
// Stores one 16x16 result block as bf16 with one dword store per lane and row
// pair: lane l holds column c = l%16 of rows 4*(l/16) + q; lanes l and l^1 swap
// two values so that the even lane writes columns (c, c+1) of rows q = 0, 1 and
// the odd lane columns (c-1, c) of rows q = 2, 3.  row_ptr(m) is the bf16 row
// of tile row m (m < rows only); col0 is the block's first column (even).
template <typename RowPtr>
__device__ __forceinline__ void store_block_bf16(const float (&v)[4], int lane, int m0, int rows,
                                                 int col0, RowPtr row_ptr) {
    const bool odd = lane & 1;
    const float s0 = odd ? v[0] : v[2], s1 = odd ? v[1] : v[3];
    // quad_perm [1, 0, 3, 2]: value of lane l^1
    const float r0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s0), 0xB1, 0xF, 0xF, false));
    const float r1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s1), 0xB1, 0xF, 0xF, false));
    const int col = col0 + ((lane & 15) & ~1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = odd ? 2 + i : i;
        const int m = m0 + (lane >> 4) * 4 + q;
        const float own = odd ? (i ? v[3] : v[2]) : (i ? v[1] : v[0]);
        const float other = i ? r1 : r0;
        if (m < rows) {
            const uint32_t pair = odd ? pack_bf16x2(other, own) : pack_bf16x2(own, other);
            *reinterpret_cast<uint32_t*>(row_ptr(m) + col) = pair;
        }
    }
}

template <int NBW, int MB>
__device__ __forceinline__ void gateup_tile(uint8_t* s_stage, int I, int wave, int lane,
                                            const TileSrc<2, NBW>& ts, int rows,
                                            int rowbase, int nbase, uint16_t* __restrict__ h) {
    f32x4 acc[MB][2][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc[mb][m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile_kloop<2, NBW, MB>(s_stage, wave, lane, ts, acc);
    // epilogue: h = silu(gate) * up, bf16, expert-sorted rows
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = silu(acc[mb][0][nb][q]) * acc[mb][1][nb][q];
            store_block_bf16(v, lane, mb * 16, rows, nbase + nb * 16,
                             [&](int m) { return h + (size_t)(rowbase + m) * I; });
        }
}

template <int NBW, int MB>
__device__ __forceinline__ void down_tile(uint8_t* s_stage, int H, int wave, int lane,
                                          const TileSrc<1, NBW>& ts, int rows,
                                          int nbase, const int* s_dst, const float* s_w,
                                          uint16_t* __restrict__ y) {
    f32x4 acc[MB][1][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[mb][0][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile_kloop<1, NBW, MB>(s_stage, wave, lane, ts, acc);
    // epilogue: the routing-weighted row, rounded to bf16, into its own row of y
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = min(mb * 16 + (lane >> 4) * 4 + q, rows - 1);
                v[q] = s_w[m] * acc[mb][0][nb][q];
            }
            store_block_bf16(v, lane, mb * 16, rows, nbase + nb * 16,
                             [&](int m) { return y + (size_t)s_dst[m] * H; });
        }
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU
// ---------------------------------------------------------------------------
template <int NBW>
__global__ __launch_bounds__(kThreads, kWgPerCu) void k_grouped_gateup(
    const uint16_t* __restrict__ x, int T, int H, int I, int E, int k,
    W4Set routed, W4Set shared, int has_shared,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    uint16_t* __restrict__ h, uint32_t* ctl) {
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[kStages * kStageBytes];
    extern __shared__ int s_pre[];       // M-tile prefix over the segments in sequence order (nseg + 1)
    __shared__ int s_tok[kBM];
    __shared__ int s_next;

    const int nseg = E + (has_shared ? 1 : 0);
    const int n_mt = build_mtile_prefix(offsets, E, T, k, has_shared, s_pre,
                                        reinterpret_cast<int*>(s_stage));   // scan scratch in the ring
    constexpr int BN = kWaves * 16 * NBW;
    const int NT = I / BN;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)uniform32(threadIdx.x / kWave);
    TileQueue tq{(int)(blockIdx.x & 7), 0u, 0u};    // thread 0's scheduling state
    uint32_t* const qb = ctl + kCtlQueueGateUp;

    if (threadIdx.x == 0) s_next = tq.next(qb, n_mt, NT);
    __syncthreads();
    for (int i = (int)uniform32(s_next); i >= 0; i = (int)uniform32(s_next)) {
        int pos, mt, nt;
        tile_coords(i, NT, s_pre, nseg, lane, pos, mt, nt);
        const TileCtx c = locate(pos, mt, s_pre, E, T, k, has_shared, offsets);
        const W4Set& Wset = c.shared ? shared : routed;
        __syncthreads();                 // previous tile's readers are done
        for (int r = threadIdx.x; r < c.rows; r += kThreads)
            s_tok[r] = c.shared ? (c.m0 + r) : min(max(perm[c.hbase + c.m0 + r], 0), T * k - 1) / k;
        __syncthreads();
        if (threadIdx.x == 0) ++tq.ran;
        const int nbase = nt * BN + wave * 16 * NBW;

        TileSrc<2, NBW> ts;
        ts.a_base = uniform64((uint64_t)x);
        const int last = c.rows - 1;
        a_offsets(ts.a_off, wave, lane, (uint32_t)H * 2u, [&](int r) { return s_tok[min(r, last)]; });
        const W4 mats[2] = {Wset.gate, Wset.up};
        uint32_t rowblk[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) rowblk[nb] = uniform32((uint32_t)(c.e * I + nbase + nb * 16));
        b_addressing(ts, mats, rowblk, H, lane);

        const int rowbase = c.hbase + c.m0;
        switch ((c.rows + 15) >> 4) {
            case 1: gateup_tile<NBW, 1>(s_stage, I, wave, lane, ts, c.rows, rowbase, nbase, h); break;
            case 2: gateup_tile<NBW, 2>(s_stage, I, wave, lane, ts, c.rows, rowbase, nbase, h); break;
            case 3: gateup_tile<NBW, 3>(s_stage, I, wave, lane, ts, c.rows, rowbase, nbase, h); break;
            case 4: gateup_tile<NBW, 4>(s_stage, I, wave, lane, ts, c.rows, rowbase, nbase, h); break;
            default: gateup_tile<NBW, kMB>(s_stage, I, wave, lane, ts, c.rows, rowbase, nbase, h); break;
        }
        if (threadIdx.x == 0) s_next = tq.next(qb, n_mt, NT);
        __syncthreads();
    }
    report_exit(ctl, kCtlExitGateUp, tq.ran, (uint32_t)(n_mt * NT));
}

// ---------------------------------------------------------------------------
// down + routing-weighted per-(token, slot) rows
// ---------------------------------------------------------------------------
template <int NBW>
__global__ __launch_bounds__(kThreads, kWgPerCu) void k_grouped_down(
    int T, int H, int I, int E, int k, W4Set routed, W4Set shared, int has_shared,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const uint16_t* __restrict__ h, uint16_t* __restrict__ y,
    uint32_t* ctl) {
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[kStages * kStageBytes];
    extern __shared__ int s_pre[];       // M-tile prefix over the segments in sequence order (nseg + 1)
    __shared__ int s_dst[kBM];           // row of y each tile row goes to
    __shared__ float s_w[kBM];
    __shared__ int s_next;

    const int nseg = E + (has_shared ? 1 : 0);
    const int n_mt = build_mtile_prefix(offsets, E, T, k, has_shared, s_pre,
                                        reinterpret_cast<int*>(s_stage));   // scan scratch in the ring
    constexpr int BN = kWaves * 16 * NBW;
    const int NT = H / BN;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)uniform32(threadIdx.x / kWave);
    TileQueue tq{(int)(blockIdx.x & 7), 0u, 0u};    // thread 0's scheduling state
    uint32_t* const qb = ctl + kCtlQueueDown;

    if (threadIdx.x == 0) s_next = tq.next(qb, n_mt, NT);
    __syncthreads();
    for (int i = (int)uniform32(s_next); i >= 0; i = (int)uniform32(s_next)) {
        int pos, mt, nt;
        tile_coords(i, NT, s_pre, nseg, lane, pos, mt, nt);
        const TileCtx c = locate(pos, mt, s_pre, E, T, k, has_shared, offsets);
        const W4Set& Wset = c.shared ? shared : routed;
        __syncthreads();
        for (int r = threadIdx.x; r < c.rows; r += kThreads) {
            if (c.shared) { s_dst[r] = T * k + c.m0 + r; s_w[r] = 1.0f; }
            else {
                const int f = min(max(perm[c.hbase + c.m0 + r], 0), T * k - 1);
                s_dst[r] = f;
                s_w[r] = topk_w[f];
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) ++tq.ran;
        const int nbase = nt * BN + wave * 16 * NBW;
        TileSrc<1, NBW> ts;
        ts.a_base = uniform64((uint64_t)(h + (size_t)(c.hbase + c.m0) * I));
        const int last = c.rows - 1;
        a_offsets(ts.a_off, wave, lane, (uint32_t)I * 2u, [&](int r) { return min(r, last); });
        const W4 mats[1] = {Wset.down};
        uint32_t rowblk[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) rowblk[nb] = uniform32((uint32_t)(c.e * H + nbase + nb * 16));
        b_addressing(ts, mats, rowblk, I, lane);

        switch ((c.rows + 15) >> 4) {
            case 1: down_tile<NBW, 1>(s_stage, H, wave, lane, ts, c.rows, nbase, s_dst, s_w, y); break;
            case 2: down_tile<NBW, 2>(s_stage, H, wave, lane, ts, c.rows, nbase, s_dst, s_w, y); break;
            case 3: down_tile<NBW, 3>(s_stage, H, wave, lane, ts, c.rows, nbase, s_dst, s_w, y); break;
            case 4: down_tile<NBW, 4>(s_stage, H, wave, lane, ts, c.rows, nbase, s_dst, s_w, y); break;
            default: down_tile<NBW, kMB>(s_stage, H, wave, lane, ts, c.rows, nbase, s_dst, s_w, y); break;
        }
        if (threadIdx.x == 0) s_next = tq.next(qb, n_mt, NT);
        __syncthreads();
    }
    report_exit(ctl, kCtlExitDown, tq.ran, (uint32_t)(n_mt * NT));
}

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const u32x4 v) {
    acc[0] += bf16lo(v.x); acc[1] += bf16hi(v.x); acc[2] += bf16lo(v.y); acc[3] += bf16hi(v.y);
    acc[4] += bf16lo(v.z); acc[5] += bf16hi(v.z); acc[6] += bf16lo(v.w); acc[7] += bf16hi(v.w);
}

// out[t][n] = bf16(sum_j y[t*k + j][n] + y[T*k + t][n]), eight columns per thread:
// the k slot rows of a token are adjacent, so every read is a 16-byte load.
// Workgroup 0 also clears both GEMMs' queue and exit words: both kernels have
// finished, so the next call finds them zero whatever state this one found.
__global__ __launch_bounds__(256) void k_finalize(const uint16_t* __restrict__ y,
                                                  uint16_t* __restrict__ out, int T, int H, int k,
                                                  int has_shared, uint32_t* ctl) {
    if (blockIdx.x == 0 && threadIdx.x < 20) {
        const int i = threadIdx.x;
        const int word = i < 8    ? kCtlQueueGateUp + i * kCtlQueueStride
                         : i < 16 ? kCtlQueueDown + (i - 8) * kCtlQueueStride
                                  : (i < 18 ? kCtlExitGateUp + (i - 16) : kCtlExitDown + (i - 18));
        __hip_atomic_store(ctl + word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const long n8 = (long)T * H / 8;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
        const long t = i / (H / 8);
        const int col = (int)(i - t * (H / 8)) * 8;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const uint16_t* row = y + (size_t)t * k * H + col;
        for (int j = 0; j < k; ++j) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(row + (size_t)j * H);
            add_bf16x8(acc, v);
        }
        if (has_shared) add_bf16x8(acc, *reinterpret_cast<const u32x4*>(y + ((size_t)T * k + t) * H + col));
        u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                   pack_bf16x2(acc[6], acc[7])};
        *reinterpret_cast<u32x4*>(out + (size_t)t * H + col) = o;
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
    const int slots = kWgPerCu * cu_count();
    const size_t pre_bytes = (size_t)(nseg + 1) * sizeof(int);
    const long gu_tiles = mt_bound * (a.I / (kWaves * 16 * NBW_GU)) + 8;
    const long dn_tiles = mt_bound * (a.H / (kWaves * 16 * NBW_DN)) + 8;
    const int g_gu = (int)(((gu_tiles < slots ? gu_tiles : slots) + 7) / 8 * 8);
    const int g_dn = (int)(((dn_tiles < slots ? dn_tiles : slots) + 7) / 8 * 8);

    tm.before();
    tm.launch(k_grouped_gateup<NBW_GU>, dim3(g_gu), dim3(kThreads), pre_bytes, st, a.x, a.T,
                       a.H, a.I, a.E, a.k, a.routed, a.shared, a.has_shared, a.offsets, a.perm,
                       a.ws_h, a.ctl);
    tm.after();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tm.before();
    tm.launch(k_grouped_down<NBW_DN>, dim3(g_dn), dim3(kThreads), pre_bytes, st, a.T, a.H, a.I,
                       a.E, a.k, a.routed, a.shared, a.has_shared, a.topk_w, a.offsets, a.perm,
                       a.ws_h, a.ws_y, a.ctl);
    tm.after();
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const long nblk = ((long)a.T * a.H / 8 + 255) / 256;
    tm.before();
    tm.launch(k_finalize, dim3((unsigned)(nblk < 4096 ? nblk : 4096)), dim3(256), 0, st,
                       a.ws_y, a.out, a.T, a.H, a.k, a.has_shared, a.ctl);
    tm.after();
    return hipGetLastError();
}

}  // namespace moe_w4
