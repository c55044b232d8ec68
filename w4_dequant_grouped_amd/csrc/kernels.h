// Host-side launch interface between the C ABI (moe_w4.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace moe_w4 {

constexpr int kSmallRouteMaxT = 8;   // largest T the one-launch router serves
constexpr int kRouterKSplit = 8;     // partial logit planes of the tiled router (T > kSmallRouteMaxT)
constexpr int kDecodeMaxT = 8;       // largest T the GEMV kernels are built for
// Largest T for which moe_w4_block runs the three-launch decode schedule (every
// routing workgroup repeats the top-k of all T rows, which stops paying off as
// the selected experts -- and workgroups -- multiply); above it, route + forward.
// Measured per layer-call against route + forward: T=3 31.9 vs 37.0 us, T=4
// 39.3 vs 42.1, T=5 56.5 vs 53.1.
constexpr int kBlockDecodeMaxT = 4;

struct W4 {                  // E matrices [N][K], packed as in moe_w4.h
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
};

struct W4Set {               // SwiGLU experts
    W4 gate, up, down;
};

struct RouteArgs {
    const uint16_t* x;
    const float* Wr;
    const float* br;
    int T, H, E, k;
    int32_t* ids;
    float* w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    float* ws_logits;        // [T][E]
    uint32_t* ws_ticket;     // control block (zero between calls)
    uint16_t* ws_planes;     // [3][E][H] bf16 split of the router weight (large T, fallback logits kernel)
    uint8_t* ws_ids8;        // [T*k] the chosen ids as bytes, padded to 16 (large T, E <= 256)
};

struct ForwardArgs {
    const uint16_t* x;
    int T, H, I, E, k;
    W4Set routed;
    W4Set shared;
    int has_shared;
    const float* topk_w;     // [T*k]
    const int32_t* offsets;  // [E+1]
    const int32_t* perm;     // [T*k]
    uint16_t* out;           // [T][H] bf16
    uint16_t* ws_h;          // [T*k + T][I] bf16: expert-sorted rows, then shared rows
    uint16_t* ws_y;          // [T*k + T][H] bf16 (grouped path): each routed (token, slot)
                             // row's weighted expert output at row t*k + j, then the
                             // shared expert's row of token t at row T*k + t
    uint32_t* ctl;           // workspace control block (zero between calls)
};

// Control block words (MOE_W4_CONTROL_BYTES / 4 of them; zero between calls
// except the error counter).
constexpr int kCtlTicket = 0;            // one-launch router: arrival ticket
constexpr int kCtlQueueStride = 32;      // 128 B between the queue words of a set
constexpr int kCtlQueueGateUp = 32;      // gate/up GEMM: 8 per-XCD tile queues
constexpr int kCtlQueueDown = kCtlQueueGateUp + 8 * kCtlQueueStride;   // down GEMM: 8 more
constexpr int kCtlExitGateUp = kCtlQueueDown + 8 * kCtlQueueStride;    // 64-bit: arrivals, tiles done
constexpr int kCtlExitDown = kCtlExitGateUp + 32;                      // 64-bit, likewise
constexpr int kCtlErrors = 1023;         // sticky count of control blocks found dirty
static_assert(kCtlExitGateUp % 2 == 0 && kCtlExitDown % 2 == 0, "64-bit exit words");
static_assert(kCtlExitDown + 2 <= kCtlErrors, "control block layout");

struct DecodeBlockArgs {     // route + forward of decode rows (T <= kDecodeMaxT)
    const uint16_t* x;
    const float* Wr;
    const float* br;
    int T, H, I, E, k;
    W4Set routed;
    W4Set shared;
    int has_shared;
    int32_t* ids;            // routing outputs, as moe_w4_route writes them
    float* tw;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    uint16_t* out;           // [T][H] bf16
    float* logits;           // [T][E] workspace
    uint16_t* h;             // [T*k + T][I] bf16 workspace
    int32_t* slots;          // [1 + 5 T k] workspace: selected experts and h rows for the down kernel
};

// Decode attention over a paged KV cache (moe_w4_attn_decode).
constexpr int kAttnMaxSplits = 256;      // partials per key/value head (combine kernel bound)

struct AttnArgs {
    const uint16_t* q;       // bf16 [Hkv*G][128]
    const uint16_t* k_pool;  // bf16 [n_pool][Hkv][64][128]
    const uint16_t* v_pool;
    const int32_t* table;    // [ceil(n_ctx / 64)]
    int n_ctx, Hkv, G, n_pool;
    int bpw;                 // blocks per workgroup (a multiple of 4)
    int nsplit;              // workgroups per key/value head
    float c;                 // softmax scale * log2(e)
    float* part_m;           // [Hkv*nsplit][16]
    float* part_l;           // [Hkv*nsplit][16]
    float* part_a;           // [Hkv*nsplit][GM][128], GM = 8 (G <= 8) or 16
    uint16_t* out;           // bf16 [Hkv*G][128]
};

// Gated DeltaNet scan (moe_w4_gdn_scan).
struct GdnArgs {
    const uint16_t* q;       // bf16 [T][Hk][128]
    const uint16_t* k;
    const uint16_t* v;       // bf16 [T][Hv][128]
    const float* g;          // [T][Hv] log decay
    const float* beta;       // [T][Hv]
    float* state;            // [Hv][128][128], read then overwritten
    uint16_t* out;           // bf16 [T][Hv][128]
    int T, Hv, Hk, rep;      // rep = Hv / Hk
};

// Chunked Gated DeltaNet scan (moe_w4_gdn_scan_chunked).  The sequence is
// processed in segments of kGdnSegT tokens (chunks of 64), each a prep launch
// over all its chunks and a scan launch; the state carries over in `state`.
constexpr int kGdnSegT = 2048;
struct GdnChunkArgs {
    const uint16_t* q;       // bf16 [T][Hk][128]
    const uint16_t* k;
    const uint16_t* v;       // bf16 [T][Hv][128]
    const float* g;          // [T][Hv]
    const float* beta;       // [T][Hv]
    float* state;            // [Hv][128][128]
    uint16_t* out;           // bf16 [T][Hv][128]
    float* ws;               // per chunk: operand fragments of one segment
    int T, Hv, Hk, rep;
    int t0, nt;              // segment: first token, tokens
};

// Optional per-kernel timing: events[2i] / events[2i+1] are recorded on the launch
// stream before / after the i-th kernel of a call (while capacity allows).
// Launches kernels and, when the caller supplies events, brackets each one with
// an event pair.  The pair is handed to hipExtLaunchKernelGGL, so the events take
// the dispatch's own begin and end timestamps (no separate event packets around
// the kernel); without events the launch is a plain one (and can be captured into
// a graph).  before() arms the next launch, after() closes the pair.
struct KernelTimer {
    hipEvent_t* events = nullptr;
    int capacity = 0;
    int count = 0;
    bool armed = false;
    void before() { armed = true; }
    void after() {
        armed = false;
        ++count;
    }
    template <typename F, typename... Args>
    void launch(F kernel, const dim3& grid, const dim3& block, uint32_t shmem, hipStream_t st,
                Args... args) {
        if (armed && events && 2 * count + 1 < capacity)
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, events[2 * count], events[2 * count + 1],
                                  0u, args...);
        else
            hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
    }
};

hipError_t launch_route_small(const RouteArgs& a, hipStream_t st, KernelTimer& tm);
hipError_t launch_route_large(const RouteArgs& a, hipStream_t st, KernelTimer& tm);
hipError_t launch_forward_decode(const ForwardArgs& a, hipStream_t st, KernelTimer& tm);
hipError_t launch_forward_grouped(const ForwardArgs& a, hipStream_t st, KernelTimer& tm);
hipError_t launch_block_decode(const DecodeBlockArgs& a, hipStream_t st, KernelTimer& tm);
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t st, KernelTimer& tm);
hipError_t launch_gdn_scan(const GdnArgs& a, hipStream_t st, KernelTimer& tm);
hipError_t launch_gdn_chunked(const GdnChunkArgs& a, hipStream_t st, KernelTimer& tm);
size_t gdn_chunked_workspace_floats(int T, int Hv, int Hk);

}  // namespace moe_w4
