// C ABI of the W4 MoE block: argument checks, workspace layout, dispatch.
// Declared and documented in include/moe_w4.h.
#include "../../include/moe_w4.h"
#include "../../include/moe_w4_attn.h"
#include "../../include/moe_w4_gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.h"

// Device scratch of moe_w4_block_noalloc(): the workspace of callers that cannot
// allocate.  Every GPU the library runs on holds its own copy until the process
// ends; static storage starts zero-filled, so its control block starts zero.
// Host code never passes this name to a kernel (on the host it stands for a
// host-side shadow, not the device copy): it uses the per-device address that
// hipGetSymbolAddress returns.
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOE_W4_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

constexpr size_t kAlign = 256;
constexpr size_t kCtrlBytes = MOE_W4_CONTROL_BYTES;
static_assert(MOE_W4_GEMV_MAX_T == moe_w4::kDecodeMaxT, "GEMV kernels are built for this many rows");

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t logits, planes, ids8, h, y, total;
};

bool dims_ok(const moe_w4_dims* d, int* status) {
    if (!d) { *status = MOE_W4_ERR_NULL; return false; }
    const uint32_t path = MOE_W4_FORWARD_GEMV | MOE_W4_FORWARD_GROUPED;
    if ((d->flags & ~path) != 0u || d->flags == path ||
        ((d->flags & MOE_W4_FORWARD_GEMV) && d->T > MOE_W4_GEMV_MAX_T)) {
        *status = MOE_W4_ERR_FLAGS;
        return false;
    }
    if (d->T < 0 || d->T > 65536 || d->E < 1 || d->E > 1024 || d->H < 256 || d->H > 16384 ||
        d->I < 128 || d->I > 16384) {
        *status = MOE_W4_ERR_DIMS;
        return false;
    }
    if (d->group != 64 || d->H % 256 != 0 || d->I % 128 != 0) { *status = MOE_W4_ERR_GROUP; return false; }
    if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->E) { *status = MOE_W4_ERR_TOPK; return false; }
    *status = MOE_W4_OK;
    return true;
}

Layout layout(const moe_w4_dims* d) {
    Layout L;
    const size_t T = (size_t)d->T, E = (size_t)d->E;
    size_t off = kCtrlBytes;
    L.logits = off;   // small T: [T][E] logits; large T: K-split partial planes
    off = align_up(off + T * E * sizeof(float) * (d->T > moe_w4::kSmallRouteMaxT ? moe_w4::kRouterKSplit : 1));
    L.planes = off;
    if (d->T > moe_w4::kSmallRouteMaxT) off = align_up(off + 3 * E * (size_t)d->H * 2);
    L.ids8 = off;     // large T: the chosen ids as bytes for the grouping kernel
    if (d->T > moe_w4::kSmallRouteMaxT) off = align_up(off + T * (size_t)d->top_k);
    L.h = off;
    off = align_up(off + (T * (size_t)d->top_k + T) * (size_t)d->I * 2);
    L.y = off;        // grouped path: per-(token, slot) output rows; decode block: slot table
    off = align_up(off + (T * (size_t)d->top_k + T) * (size_t)d->H * 2);
    L.total = off;
    return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int launch_status(hipError_t err) {
    if (err == hipSuccess) return MOE_W4_OK;
    g_last_error = hipGetErrorString(err);
    return MOE_W4_ERR_LAUNCH;
}

bool mat_ok(const moe_w4_mat& m, int* status) {
    if (!m.codes || !m.scales || !m.biases) { *status = MOE_W4_ERR_NULL; return false; }
    if (!aligned(m.codes, 16) || !aligned(m.scales, 4) || !aligned(m.biases, 4)) {
        *status = MOE_W4_ERR_ALIGN;
        return false;
    }
    return true;
}

moe_w4::W4 to_w4(const moe_w4_mat& m) { return moe_w4::W4{m.codes, m.scales, m.biases}; }

}  // namespace

extern "C" {

size_t moe_w4_workspace_bytes(const moe_w4_dims* dims) {
    int st;
    if (!dims_ok(dims, &st)) return 0;
    return layout(dims).total;
}

namespace {

int check_route(const moe_w4_dims* dims, const void* x, const float* router_w, const float* router_b,
                int32_t* topk_ids, float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                int32_t* perm, void* workspace, size_t workspace_bytes) {
    if (!x || !router_w || !topk_ids || !topk_w || !expert_counts || !expert_offsets || !perm ||
        !workspace)
        return MOE_W4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(workspace, kAlign) ||
        !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_counts, 4) ||
        !aligned(expert_offsets, 4) || !aligned(perm, 4) || (router_b && !aligned(router_b, 4)))
        return MOE_W4_ERR_ALIGN;
    if (workspace_bytes < layout(dims).total) return MOE_W4_ERR_WORKSPACE;
    return MOE_W4_OK;
}

int check_forward(const moe_w4_dims* dims, const void* x, const moe_w4_weights* routed,
                  const moe_w4_weights* shared, const float* topk_w, const int32_t* expert_offsets,
                  const int32_t* perm, void* out, void* workspace, size_t workspace_bytes) {
    if (!x || !routed || !topk_w || !expert_offsets || !perm || !out || !workspace)
        return MOE_W4_ERR_NULL;
    int st = MOE_W4_OK;
    if (!mat_ok(routed->gate, &st) || !mat_ok(routed->up, &st) || !mat_ok(routed->down, &st))
        return st;
    if (shared && (!mat_ok(shared->gate, &st) || !mat_ok(shared->up, &st) || !mat_ok(shared->down, &st)))
        return st;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, kAlign) || !aligned(topk_w, 4) ||
        !aligned(expert_offsets, 4) || !aligned(perm, 4))
        return MOE_W4_ERR_ALIGN;
    if (workspace_bytes < layout(dims).total) return MOE_W4_ERR_WORKSPACE;
    return MOE_W4_OK;
}

moe_w4::KernelTimer make_timer(void** events, int capacity) {
    moe_w4::KernelTimer tm;
    tm.events = reinterpret_cast<hipEvent_t*>(events);
    tm.capacity = events ? capacity : 0;
    return tm;
}

hipError_t run_route(const moe_w4_dims* dims, const void* x, const float* router_w,
                     const float* router_b, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* perm, void* workspace, hipStream_t stream,
                     moe_w4::KernelTimer& tm) {
    const Layout L = layout(dims);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    moe_w4::RouteArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.Wr = router_w;
    a.br = router_b;
    a.T = dims->T;
    a.H = dims->H;
    a.E = dims->E;
    a.k = dims->top_k;
    a.ids = topk_ids;
    a.w = topk_w;
    a.counts = expert_counts;
    a.offsets = expert_offsets;
    a.perm = perm;
    a.ws_ticket = reinterpret_cast<uint32_t*>(ws);
    a.ws_logits = reinterpret_cast<float*>(ws + L.logits);
    a.ws_planes = reinterpret_cast<uint16_t*>(ws + L.planes);
    a.ws_ids8 = ws + L.ids8;
    return (a.T <= moe_w4::kSmallRouteMaxT) ? moe_w4::launch_route_small(a, stream, tm)
                                            : moe_w4::launch_route_large(a, stream, tm);
}

moe_w4::W4Set to_set(const moe_w4_weights* w) {
    return moe_w4::W4Set{to_w4(w->gate), to_w4(w->up), to_w4(w->down)};
}

hipError_t run_forward(const moe_w4_dims* dims, const void* x, const moe_w4_weights* routed,
                       const moe_w4_weights* shared, const float* topk_w,
                       const int32_t* expert_offsets, const int32_t* perm, void* out,
                       void* workspace, hipStream_t stream, moe_w4::KernelTimer& tm) {
    const Layout L = layout(dims);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    moe_w4::ForwardArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.T = dims->T;
    a.H = dims->H;
    a.I = dims->I;
    a.E = dims->E;
    a.k = dims->top_k;
    a.routed = to_set(routed);
    a.has_shared = shared ? 1 : 0;
    a.shared = shared ? to_set(shared) : a.routed;
    a.topk_w = topk_w;
    a.offsets = expert_offsets;
    a.perm = perm;
    a.out = static_cast<uint16_t*>(out);
    a.ws_h = reinterpret_cast<uint16_t*>(ws + L.h);
    a.ws_y = reinterpret_cast<uint16_t*>(ws + L.y);
    a.ctl = reinterpret_cast<uint32_t*>(ws);
    const bool gemv = (dims->flags & MOE_W4_FORWARD_GEMV) ||
                      (!(dims->flags & MOE_W4_FORWARD_GROUPED) && a.T <= MOE_W4_DECODE_MAX_T);
    return gemv ? moe_w4::launch_forward_decode(a, stream, tm) : moe_w4::launch_forward_grouped(a, stream, tm);
}

}  // namespace

int moe_w4_route_timed(const moe_w4_dims* dims, const void* x, const float* router_w,
                       const float* router_b, int32_t* topk_ids, float* topk_w,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                       void* workspace, size_t workspace_bytes, void* hip_stream, void** events,
                       int capacity, int* n_kernels) {
    if (n_kernels) *n_kernels = 0;
    int st;
    if (!dims_ok(dims, &st)) return st;
    if (dims->T == 0) return MOE_W4_OK;
    st = check_route(dims, x, router_w, router_b, topk_ids, topk_w, expert_counts, expert_offsets,
                     perm, workspace, workspace_bytes);
    if (st != MOE_W4_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    moe_w4::KernelTimer tm = make_timer(events, capacity);
    const hipError_t err = run_route(dims, x, router_w, router_b, topk_ids, topk_w, expert_counts,
                                     expert_offsets, perm, workspace, stream, tm);
    if (n_kernels) *n_kernels = tm.count;
    return launch_status(err);
}

int moe_w4_route(const moe_w4_dims* dims, const void* x, const float* router_w,
                 const float* router_b, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* perm, void* workspace, size_t workspace_bytes,
                 void* hip_stream) {
    return moe_w4_route_timed(dims, x, router_w, router_b, topk_ids, topk_w, expert_counts,
                              expert_offsets, perm, workspace, workspace_bytes, hip_stream, nullptr,
                              0, nullptr);
}

int moe_w4_forward_timed(const moe_w4_dims* dims, const void* x, const moe_w4_weights* routed,
                         const moe_w4_weights* shared, const int32_t* topk_ids, const float* topk_w,
                         const int32_t* expert_offsets, const int32_t* perm, void* out,
                         void* workspace, size_t workspace_bytes, void* hip_stream, void** events,
                         int capacity, int* n_kernels) {
    (void)topk_ids;
    if (n_kernels) *n_kernels = 0;
    int st;
    if (!dims_ok(dims, &st)) return st;
    if (dims->T == 0) return MOE_W4_OK;
    st = check_forward(dims, x, routed, shared, topk_w, expert_offsets, perm, out, workspace,
                       workspace_bytes);
    if (st != MOE_W4_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    moe_w4::KernelTimer tm = make_timer(events, capacity);
    const hipError_t err = run_forward(dims, x, routed, shared, topk_w, expert_offsets, perm, out,
                                       workspace, stream, tm);
    if (n_kernels) *n_kernels = tm.count;
    return launch_status(err);
}

int moe_w4_forward(const moe_w4_dims* dims, const void* x, const moe_w4_weights* routed,
                   const moe_w4_weights* shared, const int32_t* topk_ids, const float* topk_w,
                   const int32_t* expert_offsets, const int32_t* perm, void* out, void* workspace,
                   size_t workspace_bytes, void* hip_stream) {
    return moe_w4_forward_timed(dims, x, routed, shared, topk_ids, topk_w, expert_offsets, perm, out,
                                workspace, workspace_bytes, hip_stream, nullptr, 0, nullptr);
}

int moe_w4_block_timed(const moe_w4_dims* dims, const void* x, const float* router_w,
                       const float* router_b, const moe_w4_weights* routed,
                       const moe_w4_weights* shared, int32_t* topk_ids, float* topk_w,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm, void* out,
                       void* workspace, size_t workspace_bytes, void* hip_stream, void** events,
                       int capacity, int* n_kernels) {
    if (n_kernels) *n_kernels = 0;
    int st;
    if (!dims_ok(dims, &st)) return st;
    if (dims->T == 0) return MOE_W4_OK;
    st = check_route(dims, x, router_w, router_b, topk_ids, topk_w, expert_counts, expert_offsets,
                     perm, workspace, workspace_bytes);
    if (st != MOE_W4_OK) return st;
    st = check_forward(dims, x, routed, shared, topk_w, expert_offsets, perm, out, workspace,
                       workspace_bytes);
    if (st != MOE_W4_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    moe_w4::KernelTimer tm = make_timer(events, capacity);
    if (dims->T <= moe_w4::kBlockDecodeMaxT && !(dims->flags & MOE_W4_FORWARD_GROUPED)) {
        const Layout L = layout(dims);
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        moe_w4::DecodeBlockArgs a;
        a.x = static_cast<const uint16_t*>(x);
        a.Wr = router_w;
        a.br = router_b;
        a.T = dims->T;
        a.H = dims->H;
        a.I = dims->I;
        a.E = dims->E;
        a.k = dims->top_k;
        a.routed = to_set(routed);
        a.has_shared = shared ? 1 : 0;
        a.shared = shared ? to_set(shared) : a.routed;
        a.ids = topk_ids;
        a.tw = topk_w;
        a.counts = expert_counts;
        a.offsets = expert_offsets;
        a.perm = perm;
        a.out = static_cast<uint16_t*>(out);
        a.logits = reinterpret_cast<float*>(ws + L.logits);
        a.h = reinterpret_cast<uint16_t*>(ws + L.h);
        // the decode path writes no per-slot output rows: their region holds the slot table
        a.slots = reinterpret_cast<int32_t*>(ws + L.y);
        const hipError_t err = moe_w4::launch_block_decode(a, stream, tm);
        if (n_kernels) *n_kernels = tm.count;
        return launch_status(err);
    }
    hipError_t err = run_route(dims, x, router_w, router_b, topk_ids, topk_w, expert_counts,
                               expert_offsets, perm, workspace, stream, tm);
    if (err == hipSuccess)
        err = run_forward(dims, x, routed, shared, topk_w, expert_offsets, perm, out, workspace,
                          stream, tm);
    if (n_kernels) *n_kernels = tm.count;
    return launch_status(err);
}

int moe_w4_block(const moe_w4_dims* dims, const void* x, const float* router_w,
                 const float* router_b, const moe_w4_weights* routed, const moe_w4_weights* shared,
                 int32_t* topk_ids, float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                 int32_t* perm, void* out, void* workspace, size_t workspace_bytes,
                 void* hip_stream) {
    return moe_w4_block_timed(dims, x, router_w, router_b, routed, shared, topk_ids, topk_w,
                              expert_counts, expert_offsets, perm, out, workspace, workspace_bytes,
                              hip_stream, nullptr, 0, nullptr);
}

// ---------------------------------------------------------------------------
// moe_w4_block without a caller workspace: the kernels run on the device copy of
// `scratch` of the current device.
// ---------------------------------------------------------------------------
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call made with that device current and kept for later calls.
int device_scratch(void** ptr) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return launch_status(err);
    if (dev < 0 || dev >= kMaxDevices) {
        g_last_error = "device ordinal beyond the no-allocation entry point's table";
        return MOE_W4_ERR_LAUNCH;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return launch_status(err);
        if (!p) {
            g_last_error = "hipGetSymbolAddress returned a null scratch address";
            return MOE_W4_ERR_LAUNCH;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_W4_OK;
}

}  // namespace

int moe_w4_block_noalloc(const moe_w4_dims* dims, const void* x, const float* router_w,
                         const float* router_b, const moe_w4_weights* routed,
                         const moe_w4_weights* shared, int32_t* topk_ids, float* topk_w,
                         int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                         void* out, void* hip_stream) {
    int st;
    if (!dims_ok(dims, &st)) return st;
    if (dims->T == 0) return MOE_W4_OK;
    const size_t need = layout(dims).total;
    if (need > (size_t)MOE_W4_NOALLOC_SCRATCH_BYTES) return MOE_W4_ERR_SCRATCH;
    // every argument is checked before the scratch address is looked up, with a
    // stand-in workspace pointer of the required alignment
    void* const stand_in = reinterpret_cast<void*>(kAlign);
    st = check_route(dims, x, router_w, router_b, topk_ids, topk_w, expert_counts, expert_offsets,
                     perm, stand_in, need);
    if (st != MOE_W4_OK) return st;
    st = check_forward(dims, x, routed, shared, topk_w, expert_offsets, perm, out, stand_in, need);
    if (st != MOE_W4_OK) return st;
    void* ws = nullptr;
    st = device_scratch(&ws);
    if (st != MOE_W4_OK) return st;
    return moe_w4_block_timed(dims, x, router_w, router_b, routed, shared, topk_ids, topk_w,
                              expert_counts, expert_offsets, perm, out, ws,
                              (size_t)MOE_W4_NOALLOC_SCRATCH_BYTES, hip_stream, nullptr, 0, nullptr);
}

// ---------------------------------------------------------------------------
// decode attention
// ---------------------------------------------------------------------------
namespace {

struct AttnPlan {
    int nblk, bpw, nsplit, gm;
    size_t off_l, off_a, total;
};

bool attn_dims_ok(const moe_w4_attn_dims* d, int* status) {
    if (!d) { *status = MOE_W4_ERR_NULL; return false; }
    if (d->flags != 0u) { *status = MOE_W4_ERR_FLAGS; return false; }
    if (d->n_ctx < 1 || d->n_ctx > MOE_W4_ATTN_MAX_CTX || d->n_q_heads < 1 || d->n_q_heads > 64 ||
        d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0 || d->n_q_heads / d->n_kv_heads > 16 ||
        d->n_pool_blocks < 1) {
        *status = MOE_W4_ERR_DIMS;
        return false;
    }
    if (d->head_dim != 128 || d->block != 64) { *status = MOE_W4_ERR_GROUP; return false; }
    *status = MOE_W4_OK;
    return true;
}

// Blocks per workgroup: a multiple of 4 (one per wavefront per round) chosen so
// that a key/value head has at most kAttnMaxSplits workgroups.
AttnPlan attn_plan(const moe_w4_attn_dims* d) {
    AttnPlan p;
    p.nblk = (d->n_ctx + d->block - 1) / d->block;
    const int per = (p.nblk + 4 * moe_w4::kAttnMaxSplits - 1) / (4 * moe_w4::kAttnMaxSplits);
    p.bpw = 4 * (per < 1 ? 1 : per);
    p.nsplit = (p.nblk + p.bpw - 1) / p.bpw;
    p.gm = d->n_q_heads / d->n_kv_heads <= 8 ? 8 : 16;
    const size_t parts = (size_t)d->n_kv_heads * p.nsplit;
    p.off_l = align_up(parts * 16 * sizeof(float));
    p.off_a = p.off_l + align_up(parts * 16 * sizeof(float));
    p.total = p.off_a + align_up(parts * p.gm * 128 * sizeof(float));
    return p;
}

}  // namespace

size_t moe_w4_attn_workspace_bytes(const moe_w4_attn_dims* dims) {
    int st;
    if (!attn_dims_ok(dims, &st)) return 0;
    return attn_plan(dims).total;
}

int moe_w4_attn_decode_timed(const moe_w4_attn_dims* dims, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table, void* out,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             void** events, int capacity, int* n_kernels) {
    if (n_kernels) *n_kernels = 0;
    int st;
    if (!attn_dims_ok(dims, &st)) return st;
    if (!q || !k_pool || !v_pool || !block_table || !out || !workspace) return MOE_W4_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(block_table, 4) ||
        !aligned(out, 16) || !aligned(workspace, kAlign))
        return MOE_W4_ERR_ALIGN;
    const AttnPlan p = attn_plan(dims);
    if (workspace_bytes < p.total) return MOE_W4_ERR_WORKSPACE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    moe_w4::AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_pool = static_cast<const uint16_t*>(k_pool);
    a.v_pool = static_cast<const uint16_t*>(v_pool);
    a.table = block_table;
    a.n_ctx = dims->n_ctx;
    a.Hkv = dims->n_kv_heads;
    a.G = dims->n_q_heads / dims->n_kv_heads;
    a.n_pool = dims->n_pool_blocks;
    a.bpw = p.bpw;
    a.nsplit = p.nsplit;
    a.c = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
    a.part_m = reinterpret_cast<float*>(ws);
    a.part_l = reinterpret_cast<float*>(ws + p.off_l);
    a.part_a = reinterpret_cast<float*>(ws + p.off_a);
    a.out = static_cast<uint16_t*>(out);
    moe_w4::KernelTimer tm = make_timer(events, capacity);
    const hipError_t err = moe_w4::launch_attn_decode(a, static_cast<hipStream_t>(hip_stream), tm);
    if (n_kernels) *n_kernels = tm.count;
    return launch_status(err);
}

int moe_w4_attn_decode(const moe_w4_attn_dims* dims, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, void* out,
                       void* workspace, size_t workspace_bytes, void* hip_stream) {
    return moe_w4_attn_decode_timed(dims, q, k_pool, v_pool, block_table, out, workspace,
                                    workspace_bytes, hip_stream, nullptr, 0, nullptr);
}

// ---------------------------------------------------------------------------
// Gated DeltaNet scan
// ---------------------------------------------------------------------------
int moe_w4_gdn_scan_timed(const moe_w4_gdn_dims* dims, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, float* state,
                          void* out, void* hip_stream, void** events, int capacity,
                          int* n_kernels) {
    if (n_kernels) *n_kernels = 0;
    if (!dims) return MOE_W4_ERR_NULL;
    if (dims->flags != 0u) return MOE_W4_ERR_FLAGS;
    if (dims->T < 0 || dims->T > MOE_W4_GDN_MAX_T || dims->n_v_heads < 1 || dims->n_v_heads > 128 ||
        dims->n_k_heads < 1 || dims->n_v_heads % dims->n_k_heads != 0)
        return MOE_W4_ERR_DIMS;
    if (dims->dim != 128) return MOE_W4_ERR_GROUP;
    if (dims->T == 0) return MOE_W4_OK;
    if (!q || !k || !v || !g || !beta || !state || !out) return MOE_W4_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 4) || !aligned(beta, 4) ||
        !aligned(state, 16) || !aligned(out, 16))
        return MOE_W4_ERR_ALIGN;
    moe_w4::GdnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.out = static_cast<uint16_t*>(out);
    a.T = dims->T;
    a.Hv = dims->n_v_heads;
    a.Hk = dims->n_k_heads;
    a.rep = dims->n_v_heads / dims->n_k_heads;
    moe_w4::KernelTimer tm = make_timer(events, capacity);
    const hipError_t err = moe_w4::launch_gdn_scan(a, static_cast<hipStream_t>(hip_stream), tm);
    if (n_kernels) *n_kernels = tm.count;
    return launch_status(err);
}

int moe_w4_gdn_scan(const moe_w4_gdn_dims* dims, const void* q, const void* k, const void* v,
                    const float* g, const float* beta, float* state, void* out, void* hip_stream) {
    return moe_w4_gdn_scan_timed(dims, q, k, v, g, beta, state, out, hip_stream, nullptr, 0, nullptr);
}

namespace {
int gdn_dims_status(const moe_w4_gdn_dims* dims) {
    if (!dims) return MOE_W4_ERR_NULL;
    if (dims->flags != 0u) return MOE_W4_ERR_FLAGS;
    if (dims->T < 0 || dims->T > MOE_W4_GDN_MAX_T || dims->n_v_heads < 1 || dims->n_v_heads > 128 ||
        dims->n_k_heads < 1 || dims->n_v_heads % dims->n_k_heads != 0)
        return MOE_W4_ERR_DIMS;
    if (dims->dim != 128) return MOE_W4_ERR_GROUP;
    return MOE_W4_OK;
}
}  // namespace

size_t moe_w4_gdn_chunked_workspace_bytes(const moe_w4_gdn_dims* dims) {
    if (gdn_dims_status(dims) != MOE_W4_OK) return 0;
    return moe_w4::gdn_chunked_workspace_floats(dims->T, dims->n_v_heads, dims->n_k_heads) * sizeof(float);
}

int moe_w4_gdn_scan_chunked_timed(const moe_w4_gdn_dims* dims, const void* q, const void* k,
                                  const void* v, const float* g, const float* beta, float* state,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  void* hip_stream, void** events, int capacity, int* n_kernels) {
    if (n_kernels) *n_kernels = 0;
    const int st = gdn_dims_status(dims);
    if (st != MOE_W4_OK) return st;
    if (dims->T == 0) return MOE_W4_OK;
    if (!q || !k || !v || !g || !beta || !state || !out || !workspace) return MOE_W4_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 4) || !aligned(beta, 4) ||
        !aligned(state, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return MOE_W4_ERR_ALIGN;
    if (workspace_bytes < moe_w4_gdn_chunked_workspace_bytes(dims)) return MOE_W4_ERR_WORKSPACE;
    moe_w4::GdnChunkArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.out = static_cast<uint16_t*>(out);
    a.ws = static_cast<float*>(workspace);
    a.T = dims->T;
    a.Hv = dims->n_v_heads;
    a.Hk = dims->n_k_heads;
    a.rep = dims->n_v_heads / dims->n_k_heads;
    a.t0 = 0;
    a.nt = 0;
    moe_w4::KernelTimer tm = make_timer(events, capacity);
    const hipError_t err = moe_w4::launch_gdn_chunked(a, static_cast<hipStream_t>(hip_stream), tm);
    if (n_kernels) *n_kernels = tm.count;
    return launch_status(err);
}

int moe_w4_gdn_scan_chunked(const moe_w4_gdn_dims* dims, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, float* state, void* out,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
    return moe_w4_gdn_scan_chunked_timed(dims, q, k, v, g, beta, state, out, workspace, workspace_bytes,
                                         hip_stream, nullptr, 0, nullptr);
}

const char* moe_w4_status_string(int status) {
    switch (status) {
        case MOE_W4_OK: return "ok";
        case MOE_W4_ERR_NULL: return "a required pointer is NULL";
        case MOE_W4_ERR_DIMS: return "T, H, I or E outside the supported range";
        case MOE_W4_ERR_TOPK: return "top_k must satisfy 1 <= top_k <= min(16, E)";
        case MOE_W4_ERR_GROUP: return "group must be 64, H a multiple of 256 and I a multiple of 128";
        case MOE_W4_ERR_ALIGN: return "a pointer is not aligned as required";
        case MOE_W4_ERR_WORKSPACE: return "workspace smaller than moe_w4_workspace_bytes()";
        case MOE_W4_ERR_LAUNCH: return "a HIP kernel launch failed";
        case MOE_W4_ERR_FLAGS: return "dims->flags: unknown bits, both path bits, or the GEMV path with T > 8";
        case MOE_W4_ERR_SCRATCH:
            return "the shape needs more workspace than moe_w4_block_noalloc's device scratch "
                   "(MOE_W4_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

const char* moe_w4_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
