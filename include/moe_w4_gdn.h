/*
 * Gated DeltaNet scan with the recurrent state in registers: the sequence mixer
 * of the model's linear-attention layers, on MI355X (gfx950).  Part of
 * libmoe_w4.so; status codes, error text and the timing convention are those of
 * moe_w4.h.
 *
 * Thirty of the model's 40 layers run Gated DeltaNet with a fixed-size recurrent
 * state ("Perplexity built an inference engine for one model, one chip", paragraph
 * 2), and a register-resident scan of it sped up prefill ("Perplexity's Lily brings
 * fast local AI to Apple silicon Macs", section "Where the Engine Gains Speed").
 * The recurrence is the published gated delta rule, per value head h reading
 * query/key head h / (n_v_heads / n_k_heads), for t = 0 .. T-1:
 *
 *   alpha = exp(g[t][h])
 *   S[h] <- alpha S[h] + beta[t][h] (v[t][h] - alpha S[h] k[t]) k[t]^T
 *   out[t][h] = S[h] q[t]
 *
 * Layouts (row-major, device memory owned by the caller):
 *   q, k    bf16  [T][n_k_heads][128], normalised by the caller    16-byte aligned
 *   v       bf16  [T][n_v_heads][128]                              16-byte aligned
 *   g       fp32  [T][n_v_heads]  log decay (alpha = exp(g))        4-byte aligned
 *   beta    fp32  [T][n_v_heads]                                    4-byte aligned
 *   state   fp32  [n_v_heads][128][128], state[h][i][j] = value row i, key column j;
 *           read as the initial state and overwritten with the final one  16-byte aligned
 *   out     bf16  [T][n_v_heads][128], overwritten                 16-byte aligned
 * The state stays in fp32 registers for the whole sequence; the outputs are
 * rounded once to bf16.  One kernel is enqueued on hip_stream; nothing is
 * allocated and nothing synchronises.  T == 0 is a no-op (the state is unchanged).
 *
 * Errors (nothing is enqueued when a call returns one):
 *   MOE_W4_ERR_NULL   a pointer is NULL
 *   MOE_W4_ERR_DIMS   T outside 0 .. MOE_W4_GDN_MAX_T, n_v_heads outside 1 .. 128,
 *                     n_k_heads not dividing n_v_heads
 *   MOE_W4_ERR_GROUP  dim != 128 (the size the kernel is built for)
 *   MOE_W4_ERR_ALIGN  a pointer misaligned as listed above
 *   MOE_W4_ERR_FLAGS  flags != 0
 *   MOE_W4_ERR_LAUNCH a HIP launch failed (moe_w4_last_error() has the text)
 */
#ifndef MOE_W4_GDN_H
#define MOE_W4_GDN_H

#include <stddef.h>
#include <stdint.h>

#include "moe_w4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Longest sequence one call accepts. */
#define MOE_W4_GDN_MAX_T (1 << 20)

typedef struct moe_w4_gdn_dims {
    int32_t T;           /* tokens                                 */
    int32_t n_v_heads;   /* value heads (one state each)           */
    int32_t n_k_heads;   /* query/key heads (divides n_v_heads)    */
    int32_t dim;         /* head dimension: must be 128            */
    uint32_t flags;      /* 0                                      */
} moe_w4_gdn_dims;

/* One scan over T tokens (see above). */
int moe_w4_gdn_scan(const moe_w4_gdn_dims* dims, const void* q, const void* k, const void* v,
                    const float* g, const float* beta, float* state, void* out, void* hip_stream);

/* The same, the kernel dispatched with events[0] / events[1] as its start / stop
 * events when capacity >= 2; *n_kernels receives the number of kernels enqueued. */
int moe_w4_gdn_scan_timed(const moe_w4_gdn_dims* dims, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, float* state,
                          void* out, void* hip_stream, void** events, int capacity,
                          int* n_kernels);

/*
 * The same scan computed in chunks of 64 tokens, for prefill.  Same arguments,
 * layouts, results (within rounding) and errors as moe_w4_gdn_scan(), plus a
 * device workspace of at least moe_w4_gdn_chunked_workspace_bytes(dims) bytes,
 * 16-byte aligned, owned by the caller (no initial contents are needed).
 *
 * Within a chunk the recurrence is rewritten so that only a 64 x 64 triangular
 * solve stays sequential: with G the running sum of the log decays, the chunk's
 * state corrections solve (I + A) U = diag(beta) (V - Gamma K S0^T), A[t][s] =
 * beta_t exp(G_t - G_s) k_t . k_s for s < t, and the outputs and the next state
 * are matrix products of U, S0, Q and K (the chunked form of the published
 * gated delta rule).  Products run on bf16 MFMA with fp32 accumulation; fp32
 * operands (the state, the solve's results) enter as bf16 hi + lo pairs, so the
 * state keeps about 16 significant bits per product term.  The sequence is
 * processed in segments of 2048 tokens, two kernels each; the state carries over
 * in `state`.  Errors as moe_w4_gdn_scan(), and MOE_W4_ERR_NULL for a NULL
 * workspace, MOE_W4_ERR_ALIGN for a misaligned one, MOE_W4_ERR_WORKSPACE for one
 * that is too small.
 */
size_t moe_w4_gdn_chunked_workspace_bytes(const moe_w4_gdn_dims* dims);

int moe_w4_gdn_scan_chunked(const moe_w4_gdn_dims* dims, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, float* state, void* out,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* The same with per-kernel timing events (two kernels per 2048-token segment). */
int moe_w4_gdn_scan_chunked_timed(const moe_w4_gdn_dims* dims, const void* q, const void* k,
                                  const void* v, const float* g, const float* beta, float* state,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  void* hip_stream, void** events, int capacity, int* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_GDN_H */
