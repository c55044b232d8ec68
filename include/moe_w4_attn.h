/*
 * Decode attention over a paged KV cache: the attention half of a decode step of
 * the model's full-attention layers, on MI355X (gfx950).  Part of libmoe_w4.so;
 * status codes, error text and the timing convention are those of moe_w4.h.
 *
 * One new query token attends to the n_ctx cached tokens (the cache already holds
 * the new token's key and value).  The model has 16 query heads over two
 * key/value heads ("Perplexity's Lily brings fast local AI to Apple silicon
 * Macs", section "A 35B Model Built for Local Memory").  Query head h reads cache
 * head h / G, G = n_q_heads / n_kv_heads:
 *
 *   out[h] = sum_n softmax_n( q[h] . K[h/G][n] / sqrt(head_dim) ) * V[h/G][n]
 *
 * The query heads of a group are packed so that each cached key and value row is
 * read once for all of them, and the cache is stored in fixed-size blocks found
 * through a block table ("Perplexity built an inference engine for one model, one
 * chip", paragraph 3; "Perplexity's Lily ...", section "Where the Engine Gains
 * Speed").
 *
 * Layouts (all row-major, device memory owned by the caller):
 *   q            bf16  [n_q_heads][head_dim]                          16-byte aligned
 *   k_pool       bf16  [n_pool_blocks][n_kv_heads][block][head_dim]   16-byte aligned
 *   v_pool       bf16  same as k_pool                                 16-byte aligned
 *   block_table  int32 [ceil(n_ctx / block)]: token n is slot n % block of
 *                physical block block_table[n / block]; entries outside
 *                0 .. n_pool_blocks - 1 are clamped into it (never read out of
 *                bounds).  Slots past n_ctx in the last block are never used,
 *                whatever they hold.                                  4-byte aligned
 *   out          bf16  [n_q_heads][head_dim], overwritten; fp32 softmax and sums,
 *                one round to nearest even at the end.               16-byte aligned
 *   workspace    moe_w4_attn_workspace_bytes(dims) bytes, 256-byte aligned; holds
 *                per-split partial results, needs no clearing.
 *
 * Errors (nothing is enqueued when a call returns one):
 *   MOE_W4_ERR_NULL       a pointer is NULL
 *   MOE_W4_ERR_DIMS       n_ctx outside 1 .. MOE_W4_ATTN_MAX_CTX, n_q_heads outside
 *                         1 .. 64, n_kv_heads not dividing n_q_heads, a group larger
 *                         than 16, or n_pool_blocks < 1
 *   MOE_W4_ERR_GROUP      head_dim != 128 or block != 64 (the sizes the kernels
 *                         are built for)
 *   MOE_W4_ERR_ALIGN      a pointer misaligned as listed above
 *   MOE_W4_ERR_WORKSPACE  workspace_bytes too small
 *   MOE_W4_ERR_FLAGS      flags != 0
 *   MOE_W4_ERR_LAUNCH     a HIP launch failed (moe_w4_last_error() has the text)
 * Two kernels are enqueued on hip_stream (NULL: the default stream); the library
 * allocates nothing and does not synchronise.
 */
#ifndef MOE_W4_ATTN_H
#define MOE_W4_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include "moe_w4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest context one call accepts. */
#define MOE_W4_ATTN_MAX_CTX (1 << 20)

typedef struct moe_w4_attn_dims {
    int32_t n_ctx;          /* cached tokens attended to                    */
    int32_t n_q_heads;      /* query heads                                  */
    int32_t n_kv_heads;     /* key/value heads (divides n_q_heads)          */
    int32_t head_dim;       /* must be 128                                  */
    int32_t block;          /* tokens per cache block: must be 64           */
    int32_t n_pool_blocks;  /* physical blocks in k_pool and v_pool         */
    uint32_t flags;         /* 0                                            */
} moe_w4_attn_dims;

/* Workspace bytes for these dims; 0 when the dims are invalid. */
size_t moe_w4_attn_workspace_bytes(const moe_w4_attn_dims* dims);

/* One decode-attention step (see above). */
int moe_w4_attn_decode(const moe_w4_attn_dims* dims, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, void* out,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* The same with per-kernel timing, as the *_timed calls of moe_w4.h: kernel i is
 * dispatched with events[2i] and events[2i+1] as its start and stop events while
 * 2i+1 < capacity; *n_kernels receives the number of kernels enqueued. */
int moe_w4_attn_decode_timed(const moe_w4_attn_dims* dims, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table, void* out,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             void** events, int capacity, int* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_ATTN_H */
