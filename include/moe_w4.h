/*
 * moe_w4.h -- C ABI of the MI355X (gfx950) mixture-of-experts block with
 * groupwise-affine 4-bit expert weights.
 *
 * The block: a router picks top_k of E experts per token and one shared expert
 * sees every token ("Perplexity built an inference engine for one model, one
 * chip", paragraph 2: eight of 256 experts plus one shared expert).  Expert
 * weights are groupwise-affine 4-bit ("Perplexity's Lily brings fast local AI to
 * Apple silicon Macs", section "A 35B Model Built for Local Memory") and are
 * reconstructed tile by tile inside the grouped GEMM, never written out expanded
 * (same page, section "Where the Engine Gains Speed"; "Perplexity built an
 * inference engine for one model, one chip", paragraph 3).  Routing stays on the
 * GPU: no call copies device data to the host or synchronises (same paragraph).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer except `dims`, the weight descriptors and the returned strings
 *    is a DEVICE pointer (hipMalloc'd or equivalent) on the current HIP device.
 *    The caller owns all memory; the library allocates nothing, keeps no state
 *    between calls, never copies device data to the host and never synchronises.
 *    All work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream).
 *  - Dense row-major layouts, no strides.  bf16 values travel as uint16 bit
 *    patterns.
 *  - Arguments are validated on the host before anything is launched; a negative
 *    return value means nothing was enqueued (except MOE_W4_ERR_LAUNCH, see
 *    below).  T == 0 returns MOE_W4_OK and enqueues nothing.
 *  - MOE_W4_ERR_LAUNCH: a HIP launch failed; kernels enqueued before it may
 *    still run.  moe_w4_last_error() returns the HIP message (thread-local).
 *    Device faults surface at the caller's next synchronisation, as in HIP.
 *  - Workspace: `workspace` must hold at least moe_w4_workspace_bytes(dims)
 *    bytes, be 256-byte aligned, and be ZERO-FILLED before the first call that
 *    uses it.  Its first MOE_W4_CONTROL_BYTES bytes are a control block (ticket
 *    and work-queue counters) that every call leaves zero again, except the
 *    error counter at MOE_W4_CONTROL_ERRORS_OFFSET.  route() and forward() for
 *    the same dims may share one workspace; calls that may run concurrently need
 *    distinct workspaces.
 *  - A dirty control block is detected, counted and repaired where it matters
 *    most: the grouped GEMMs of forward() (T > MOE_W4_DECODE_MAX_T) count the
 *    tiles they run; a call that ran fewer than its tile list holds, or met
 *    arrival counts past its grid, adds one to the error counter, and its last
 *    kernel clears every work-queue word, so the next call starts clean.  (The
 *    output of the call that found the block dirty is unspecified.)  The
 *    one-launch router (route() for T <= 8) counts an arrival ticket beyond its
 *    grid as an error and clears the ticket.
 *
 * Weight layout (moe_w4_mat), for E matrices of shape [N][K]:
 *    codes   uint8  [E][N][K/2]   byte j of a row holds k = 2j in bits 0..3 and
 *                                 k = 2j+1 in bits 4..7; codes are unsigned 0..15
 *    scales  bf16   [E][N][K/G]   per (row, group of G consecutive k)
 *    biases  bf16   [E][N][K/G]
 *    dequantised weight  w[e][n][k] = code * scale[e][n][k/G] + bias[e][n][k/G]
 *  `codes` must be 16-byte aligned, `scales` and `biases` 4-byte aligned.
 *  `x`, `out` and `router_w` must be 16-byte aligned, int32/fp32 arrays 4-byte.
 *
 * Supported sizes (checked): 1 <= top_k <= 16, top_k <= E <= 1024, group == 64,
 * H % 256 == 0, I % 128 == 0, 0 <= T <= 65536, H, I <= 16384.
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest T served by the decode (GEMV) path of moe_w4_forward() by default:
 * the measured crossover with the grouped path on MI355X for H=2048, I=512,
 * E=256, top-8 (the GEMV path is faster through T=7, the grouped path from 8). */
#define MOE_W4_DECODE_MAX_T 7

/* Largest T the decode (GEMV) path accepts when it is chosen explicitly. */
#define MOE_W4_GEMV_MAX_T 8

/* dims->flags: which forward path runs.  0 chooses by T (the GEMV path for
 * T <= MOE_W4_DECODE_MAX_T, the grouped MFMA path above).  MOE_W4_FORWARD_GEMV
 * forces the GEMV path (T <= MOE_W4_GEMV_MAX_T); MOE_W4_FORWARD_GROUPED forces the
 * grouped path at any T (moe_w4_block then also skips its single-call schedule).
 * Both bits, any other bit, or MOE_W4_FORWARD_GEMV with a larger T is
 * MOE_W4_ERR_FLAGS.  Routing does not depend on the bits; route() accepts them so
 * that one dims struct serves route() and forward(). */
#define MOE_W4_FORWARD_GEMV 1u
#define MOE_W4_FORWARD_GROUPED 2u

/* Bytes at the start of the workspace used as the control block. */
#define MOE_W4_CONTROL_BYTES 4096

/* Byte offset, within the control block, of a uint32 counter of calls that found
 * the control block dirty (not zero-filled, or shared with a concurrent call).
 * The library only ever increments it; the caller may read or clear it. */
#define MOE_W4_CONTROL_ERRORS_OFFSET 4092

enum {
    MOE_W4_OK = 0,
    MOE_W4_ERR_NULL = -1,        /* a required pointer is NULL                     */
    MOE_W4_ERR_DIMS = -2,        /* T, H, I or E out of the supported range         */
    MOE_W4_ERR_TOPK = -3,        /* top_k < 1, > 16 or > E                          */
    MOE_W4_ERR_GROUP = -4,       /* group != 64, or H / I not a multiple it needs   */
    MOE_W4_ERR_ALIGN = -5,       /* a pointer is not aligned as documented          */
    MOE_W4_ERR_WORKSPACE = -6,   /* workspace smaller than moe_w4_workspace_bytes() */
    MOE_W4_ERR_LAUNCH = -7,      /* a HIP launch failed (see moe_w4_last_error())   */
    MOE_W4_ERR_FLAGS = -8,       /* bad dims->flags (see MOE_W4_FORWARD_GEMV)        */
    MOE_W4_ERR_SCRATCH = -9      /* shape too large for moe_w4_block_noalloc()      */
};

/* Size of the device scratch that moe_w4_block_noalloc() uses in place of a
 * workspace (32 MiB per GPU). */
#define MOE_W4_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Sizes of one block call.  `flags`: 0, or one forward-path bit (above). */
typedef struct moe_w4_dims {
    int32_t T;       /* tokens: rows of x and of out                    */
    int32_t H;       /* hidden size                                     */
    int32_t I;       /* intermediate size of every expert (and shared)  */
    int32_t E;       /* routed experts                                  */
    int32_t top_k;   /* experts chosen per token                        */
    int32_t group;   /* quantisation group along K (must be 64)         */
    uint32_t flags;  /* 0 or MOE_W4_FORWARD_GEMV / MOE_W4_FORWARD_GROUPED */
} moe_w4_dims;

/* Packed 4-bit weights of E matrices [N][K] (layout above). */
typedef struct moe_w4_mat {
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
} moe_w4_mat;

/* One set of SwiGLU experts: gate and up are [E][I][H], down is [E][H][I]. */
typedef struct moe_w4_weights {
    moe_w4_mat gate;
    moe_w4_mat up;
    moe_w4_mat down;
} moe_w4_weights;

/*
 * Bytes of device workspace route() and forward() need for `dims` (0 if the
 * dims are invalid).  Pure host function.
 */
size_t moe_w4_workspace_bytes(const moe_w4_dims* dims);

/*
 * Route T tokens on the GPU ("Perplexity built an inference engine for one
 * model, one chip", paragraphs 2 and 3: the router picks eight of 256 experts,
 * and routing never goes back to the CPU).
 *
 *   x            bf16  [T][H]     activations
 *   router_w     fp32  [E][H]     router weight
 *   router_b     fp32  [E]        additive per-expert logit bias, or NULL
 * outputs (overwritten):
 *   topk_ids     int32 [T][top_k] chosen experts of each token, ascending id
 *   topk_w       fp32  [T][top_k] weight of topk_ids[t][j]: softmax over all E
 *                                 logits, renormalised over the chosen top_k
 *   expert_counts  int32 [E]      tokens routed to each expert
 *   expert_offsets int32 [E+1]    exclusive prefix sum of expert_counts
 *   perm         int32 [T*top_k]  the values t*top_k + j, ordered by
 *                                 (expert topk_ids[t][j], then t)
 * Logits are l = x W_r^T + b_r in fp32.  The top_k largest logits are chosen,
 * ties going to the lower expert index.
 */
int moe_w4_route(const moe_w4_dims* dims,
                 const void* x, const float* router_w, const float* router_b,
                 int32_t* topk_ids, float* topk_w,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                 void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Block output for routed tokens:
 *   out[t] = sum_j topk_w[t][j] * FFN_{topk_ids[t][j]}(x[t]) + FFN_shared(x[t])
 *   FFN(v) = Wd (silu(Wg v) * (Wu v)),  silu(z) = z / (1 + exp(-z))
 * with every W the dequantised 4-bit matrix ("Perplexity's Lily brings fast
 * local AI to Apple silicon Macs", section "Where the Engine Gains Speed": the
 * weights are reconstructed inside the grouped GEMM one tile at a time).
 *
 *   x            bf16  [T][H]
 *   routed       E experts' weights (descriptor in host memory, pointers on device)
 *   shared       one expert's weights, or NULL for no shared expert
 *   topk_w, expert_offsets, perm   as produced by moe_w4_route() for this x
 *   out          bf16  [T][H]     overwritten; must not alias x
 * T <= MOE_W4_DECODE_MAX_T (or dims->flags) selects the decode path (one wavefront per weight row
 * streams each selected expert's bytes once); larger T runs the grouped MFMA
 * path.  Both accumulate in fp32; intermediate activations are rounded to bf16.
 * The grouped path rounds each routed (token, slot) row's weighted expert output
 * and the shared expert's output to bf16, then sums a token's rows in fp32 in
 * slot order (shared last), so its result does not depend on scheduling.
 * perm must be a permutation of 0 .. T*top_k-1 consistent with expert_offsets, as
 * route() writes it: other values cannot make an access leave its buffer, but
 * the output is then unspecified.
 * `topk_ids` is accepted for interface symmetry and may be NULL.
 */
int moe_w4_forward(const moe_w4_dims* dims, const void* x,
                   const moe_w4_weights* routed, const moe_w4_weights* shared,
                   const int32_t* topk_ids, const float* topk_w,
                   const int32_t* expert_offsets, const int32_t* perm,
                   void* out, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * moe_w4_route() followed by moe_w4_forward() in one call, with the same
 * arguments, outputs and errors as the pair: every argument is validated before
 * anything is enqueued.  The routing outputs are written as moe_w4_route()
 * writes them.  For T <= 4 the work is scheduled as three kernels instead of the
 * pair's: (1) router logits together with the shared expert's gate/up, which
 * need only x; (2) top-k and grouping repeated by every workgroup from the
 * logits, followed by the selected experts' gate/up; (3) down and the weighted
 * combine.  Splitting the decode step so that independent reads stream together
 * and no single workgroup serialises the routing follows the pages' emphasis on
 * the hand-off between decode stages ("Perplexity's Lily brings fast local AI
 * to Apple silicon Macs", section "Where the Engine Gains Speed").  For larger
 * T it enqueues route then forward.
 */
int moe_w4_block(const moe_w4_dims* dims, const void* x,
                 const float* router_w, const float* router_b,
                 const moe_w4_weights* routed, const moe_w4_weights* shared,
                 int32_t* topk_ids, float* topk_w,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                 void* out, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * The same calls with per-kernel timing.  When `events` is not NULL it holds
 * `capacity` hipEvent_t handles created by the caller; the i-th kernel the call
 * launches (while 2i+1 < capacity) is dispatched with events[2i] and
 * events[2i+1] as its start and stop events (hipExtLaunchKernelGGL), so
 * hipEventElapsedTime on the pair gives that kernel's own execution time.
 * *n_kernels (if not NULL) receives the number of kernels launched.  Everything
 * else is as for moe_w4_route() and moe_w4_forward().
 */
int moe_w4_route_timed(const moe_w4_dims* dims,
                       const void* x, const float* router_w, const float* router_b,
                       int32_t* topk_ids, float* topk_w,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                       void* workspace, size_t workspace_bytes, void* hip_stream,
                       void** events, int capacity, int* n_kernels);

int moe_w4_forward_timed(const moe_w4_dims* dims, const void* x,
                         const moe_w4_weights* routed, const moe_w4_weights* shared,
                         const int32_t* topk_ids, const float* topk_w,
                         const int32_t* expert_offsets, const int32_t* perm,
                         void* out, void* workspace, size_t workspace_bytes, void* hip_stream,
                         void** events, int capacity, int* n_kernels);

int moe_w4_block_timed(const moe_w4_dims* dims, const void* x,
                       const float* router_w, const float* router_b,
                       const moe_w4_weights* routed, const moe_w4_weights* shared,
                       int32_t* topk_ids, float* topk_w,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                       void* out, void* workspace, size_t workspace_bytes, void* hip_stream,
                       void** events, int capacity, int* n_kernels);

/*
 * moe_w4_block() for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs and errors as moe_w4_block() without `workspace` and
 * `workspace_bytes`: the kernels use a device scratch array of
 * MOE_W4_NOALLOC_SCRATCH_BYTES bytes that the library holds, one copy per GPU,
 * until the process ends.  The caller still passes every input and output.
 *  - Shapes whose moe_w4_workspace_bytes() exceeds MOE_W4_NOALLOC_SCRATCH_BYTES
 *    return MOE_W4_ERR_SCRATCH and enqueue nothing (at H=2048, I=512, E=256,
 *    top-8 with a shared expert that is T <= 560).
 *  - The call allocates nothing: no hipMalloc, no hipFree, no allocating library
 *    routine.  The first call with a given device current looks up that device's
 *    scratch address (hipGetSymbolAddress) and keeps it.
 *  - Every call on one GPU shares that GPU's scratch, which keeps the last
 *    call's contents; its control block starts zero-filled and every call leaves
 *    it zero.  Calls that may overlap on one GPU (other streams, other host
 *    threads) race on the scratch: serialise them, or use moe_w4_block() with
 *    distinct workspaces.
 */
int moe_w4_block_noalloc(const moe_w4_dims* dims, const void* x,
                         const float* router_w, const float* router_b,
                         const moe_w4_weights* routed, const moe_w4_weights* shared,
                         int32_t* topk_ids, float* topk_w,
                         int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                         void* out, void* hip_stream);

/* Static description of a status code. */
const char* moe_w4_status_string(int status);

/* Message of the last failing HIP call on this thread ("" if none). */
const char* moe_w4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_H */
