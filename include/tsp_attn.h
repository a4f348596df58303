/*
 * tsp_attn.h -- C ABI of one rank's attention block under tensor-and-sequence
 * parallel (TSP) sharding, on MI355X (gfx950). Same library, status codes,
 * error conventions and tsp_last_error() as tsp_mlp.h.
 *
 * What the library computes
 * -------------------------
 * "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
 * Training & Inference", Abstract: every rank holds one parameter shard and
 * one sequence shard; for attention the ranks go through the broadcast
 * parameter shards one after another and rebuild the full context with a
 * sequence-wise exchange of keys and values. "Tensor Parallelism: Splitting
 * the Math", section "Why the column-then-row split - and what happens in
 * attention": heads are independent, so the Q, K, V projections split by
 * columns (whole heads) and the output projection by the matching rows.
 * "Tensor Parallelism" (AI terminology page), table "Key Points", row
 * "Attention split": a shard is a contiguous range of heads.
 *
 * A sequence of S = P T tokens is split into P contiguous shards; rank r owns
 * positions [r T, (r + 1) T). Head group s (s = 0..P-1) owns query heads
 * [s H/P, (s+1) H/P) and key/value heads [s Hkv/P, (s+1) Hkv/P). For the
 * rank's tokens X (T x d):
 *
 *   Y = sum_{k=0..P-1} O_{order[k]} . Wo[rows of group order[k], :]
 *   O_s = per head h of group s: softmax(Q_h K_j^T / sqrt(dh) + mask) V_j,
 *         j = h / (H / Hkv) (grouped key/value heads)
 *   Q_h = X . Wq[:, h dh .. (h+1) dh),  K_j, V_j = every rank's X . Wk / Wv
 *         columns of head j (the exchanged context, positions 0..S-1)
 *
 * The mask hides keys at positions after the query's own (causal) when the
 * handle is causal; otherwise every key is visible. No biases, no position
 * encoding. Q, K, V and the probabilities are rounded to fp16 (nearest
 * even, 11 significant bits) where the kernels store or multiply them, O to
 * bf16 (like the MLP's hidden activations) before the output projection;
 * scores, softmax sums and Y accumulate in fp32. Y is fp32 and overwritten.
 * fp16 bounds the projections: an entry of X Wq / sqrt(dh) log2(e), X Wk or
 * X Wv beyond 65504 in magnitude becomes infinite and the output NaN.
 *
 * The exchange on one GPU: the handle owns the context, keys and values of
 * all S positions for every key/value head. tsp_attn_project_kv(rank rho)
 * writes rank rho's rows (what rho itself computes and sends);
 * tsp_attn_forward(rank r) writes rank r's own rows first, then reads the
 * rows of every rank it attends to (ranks 0..r when causal, all when not).
 * Those rows must have been written by tsp_attn_project_kv with the same T
 * since T last changed; rows never written read as zero.
 *
 * Context layout (library-owned): K as positions x (Hkv dh); V transposed,
 * (Hkv dh) x positions, each 32-position group stored as 4 chunks of 8 where
 * chunk j holds positions 4j..4j+3 and 16+4j..16+4j+3 of the group.
 *
 * Layouts: row-major, no padding; X is T x d bf16, Y is T x d fp32, w_q is
 * d x (H dh), w_k and w_v are d x (Hkv dh), w_o is (H dh) x d (Y = X W,
 * input x output); head h occupies columns [h dh, (h+1) dh).
 *
 * Shapes the kernels take (else TSP_ERR_UNSUPPORTED): bf16 only; dh = 128;
 * P divides Hkv and Hkv divides H; H / Hkv is 1, 2 or a multiple of 4;
 * H / P even; d a multiple of 256; T a multiple of 32.
 */
#ifndef TSP_ATTN_H
#define TSP_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "tsp_mlp.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tsp_attn* tsp_attn_t;   /* opaque */

/*
 * Packs head group order[k]'s columns of w_q, w_k, w_v and rows of w_o as
 * record k (order: P entries, a permutation of 0..P-1, the rank's visiting
 * order, e.g. (r + k) mod P for rank r; NULL = 0..P-1), allocates the context
 * for P * T_max positions (zeroed) and the workspace, and synchronises
 * `stream` before returning: the caller may then free its weights. Weight
 * pointers are device pointers, 16-byte aligned. On failure *out is NULL and
 * nothing is leaked (TSP_ERR_OOM when device memory runs out).
 */
tsp_status_t tsp_attn_create(tsp_attn_t* out, int64_t T_max, int64_t d, int32_t H, int32_t Hkv, int32_t dh,
                             int32_t P, int32_t causal, const int32_t* order, const void* w_q, const void* w_k,
                             const void* w_v, const void* w_o, hipStream_t stream);

/*
 * The exchange stand-in: projects rank `rank`'s T tokens X (T x d bf16,
 * device) through every head group's K and V columns into the handle's
 * context rows [rank T, (rank + 1) T). Asynchronous on `stream` (NULL = the
 * create stream). 0 <= rank < P, 1 <= T <= T_max, T a multiple of 32.
 */
tsp_status_t tsp_attn_project_kv(tsp_attn_t h, int64_t T, int32_t rank, const void* X, hipStream_t stream);

/*
 * Rank `rank`'s forward: Y (T x d fp32, device, overwritten) from its tokens
 * X (T x d bf16, device): the Q/K/V projection of X (its K and V rows land
 * in the context), attention over the context, and the output projection,
 * head group by head group in the handle's order. Asynchronous on `stream`;
 * one forward or projection in flight per handle (they share the workspace
 * and the context). Y must not overlap X. It only launches kernels on
 * `stream` (with kernel timing off), so it can be captured into a HIP graph
 * and replayed.
 */
tsp_status_t tsp_attn_forward(tsp_attn_t h, int64_t T, int32_t rank, const void* X, float* Y,
                              hipStream_t stream);

/* Synchronises the handle's stream and frees everything; NULL is a no-op. */
tsp_status_t tsp_attn_destroy(tsp_attn_t h);

/* Per-kernel HIP-event timing, as tsp_mlp_set_timing / tsp_mlp_read_timing:
 * kernels attn_qkv, attn_core, attn_out (and reduce_partials when the output
 * projection is split into ring groups). */
tsp_status_t tsp_attn_set_timing(tsp_attn_t h, int32_t enable);
tsp_status_t tsp_attn_read_timing(tsp_attn_t h, int32_t max_kernels, char (*names)[64], double* total_ms,
                                  int64_t* launches, int32_t* n_kernels);

/* Bytes of the packed weights, workspace and context the handle holds. */
tsp_status_t tsp_attn_sizes(tsp_attn_t h, int64_t* packed_bytes, int64_t* workspace_bytes, int64_t* context_bytes);

#ifdef __cplusplus
}
#endif

#endif /* TSP_ATTN_H */
