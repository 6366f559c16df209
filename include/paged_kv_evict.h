/*
 * paged_kv_evict.h -- C-ABI of the PagedEviction part of the MI355X (gfx950)
 * paged KV cache library: token importance over the paged cache, the
 * decode-phase eviction of whole blocks, and the prefill-phase compression
 * of each sequence to a token budget.
 *
 * The method (page "KV缓存内存布局优化：分页策略、量化压缩与动态驱逐的工程实践",
 * blog.hotdry.top, section "PagedEviction 块级驱逐机制"): a token's importance
 * is the ratio of the L2 norms of its value and key, S_t = ||V_t|| / ||K_t||,
 * computed without attention scores; during decode, when the newest block of
 * a sequence fills, the mean importance of each existing full block is
 * evaluated and the full block with the lowest mean is evicted whole, which
 * keeps every block full and the layout regular.
 *
 * Readings taken here: K_t and V_t are the token's whole rows in one layer's
 * cache (all kv heads, all dims, dequantized for int8 / fp8); a token's score
 * lives with its slot, like its K/V (scores[block * block_size + slot]), so an
 * eviction moves only block ids.
 *
 * Layouts (row-major; all pointers are DEVICE memory owned by the caller):
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim]: bf16,
 *                     int8 (+ k_scales / v_scales fp32 [num_blocks,
 *                     block_size, num_kv_heads]) or FP8 E4M3 codes, exactly as
 *                     for paged_attn_decode*
 *   block_tables      int32 [num_seqs, max_blocks_per_seq]
 *   token_begin       int32 [num_seqs] or NULL (= 0 for every sequence)
 *   context_lens      int32 [num_seqs]
 *   scores            fp32 [num_blocks, block_size]
 *   evict_mask        int32 [num_seqs]; evicted int32 [num_seqs]
 *
 * Ownership and state: the library allocates nothing and keeps no state.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 * Errors: PA_OK or a negative PA_ERR_* code of paged_attn.h, detected on the
 * host before any launch (nothing is written then).  Not checked (it would
 * need a device read): context_lens[s] <= max_blocks_per_seq * block_size and
 * valid block ids for every block the context uses; token_begin[s] >= 0.
 */
#ifndef PAGED_KV_EVICT_H
#define PAGED_KV_EVICT_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_score_shape {
    int32_t num_seqs;           /* S >= 0 (0 is a no-op) */
    int32_t num_kv_heads;       /* Hkv >= 1 */
    int32_t head_dim;           /* 64 or 128 */
    int32_t block_size;         /* tokens per block, 1 .. 4096 */
    int32_t max_blocks_per_seq; /* row length of block_tables, >= 1 */
    int32_t num_blocks;         /* blocks in the pool, >= 1 */
} pa_score_shape;

/*
 * Importance of tokens [token_begin[s], context_lens[s]) of every sequence:
 * scores[b * block_size + r] = ||V|| / ||K|| for the token in physical block
 * b, slot r (fp32: squares summed in fp32, IEEE square roots and division).
 * A key row of zeros gives +inf (0/0 gives NaN).  Other score entries are not
 * written.  The bf16, int8 and fp8 forms read the cache like the decode entry
 * points; k_cache / v_cache 16-byte aligned (bf16) or 8-byte aligned.  One
 * kernel launch.
 */
int paged_kv_token_scores(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                          const int32_t *token_begin, const int32_t *context_lens, float *scores,
                          const pa_score_shape *shape, void *stream);

int paged_kv_token_scores_int8(const int8_t *k_cache, const int8_t *v_cache,
                               const float *k_scales, const float *v_scales,
                               const int32_t *block_tables, const int32_t *token_begin,
                               const int32_t *context_lens, float *scores,
                               const pa_score_shape *shape, void *stream);

int paged_kv_token_scores_fp8(const uint8_t *k_cache, const uint8_t *v_cache,
                              const int32_t *block_tables, const int32_t *token_begin,
                              const int32_t *context_lens, float *scores,
                              const pa_score_shape *shape, void *stream);

/*
 * Decode-phase block eviction.  For each sequence s with evict_mask[s] != 0
 * and at least one full block (context_lens[s] / block_size > 0):
 *   - the mean of full block j is the sum, in double and in slot order, of
 *     its block_size scores, divided by block_size;
 *   - the victim is the full block of smallest mean (lowest j among equal
 *     means; a NaN mean is never chosen unless all are NaN, then block 0);
 *   - block_tables[s][j+1 .. nblk-1] move down one entry, entry nblk-1
 *     becomes -1 (nblk = ceil(context_lens[s] / block_size)),
 *     context_lens[s] -= block_size, and evicted[s] receives the victim's
 *     physical block id, which the caller may reuse.
 * Other sequences get evicted[s] = -1 and are left unchanged.  block_tables
 * and context_lens are updated in place; scores are only read.  One kernel
 * launch.
 */
int paged_kv_evict_lowest_block(const float *scores, int32_t *block_tables,
                                int32_t *context_lens, const int32_t *evict_mask,
                                int32_t *evicted, const pa_score_shape *shape, void *stream);

/*
 * Prefill-phase token compression (same page and section: in the prefill
 * phase the tokens of low importance are evicted until the cache holds the
 * budget).  For each sequence s with n = context_lens[s] > budget:
 *   - tokens are ranked by their importance scores[slot] (as written by
 *     paged_kv_token_scores*): highest first, a NaN above every number, equal
 *     values (-0 and +0 included) by position, earlier first;
 *   - the first `budget` tokens of that ranking are kept, in their original
 *     order, and move to logical positions 0 .. budget-1 of the same
 *     sequence: each takes its K and V rows (all kv heads), its int8 scales
 *     and its importance with it;
 *   - context_lens[s] becomes budget.
 * Sequences with n <= budget, slots at positions >= budget and the block
 * tables are left unchanged; table entries from ceil(budget / block_size) on
 * no longer belong to the context, and the caller may reuse their blocks.
 * k_cache, v_cache (and the scales, and scores) are updated in place, and
 * must be 16-byte aligned.
 *
 * Workspace: paged_kv_compress_workspace_bytes(shape, budget) bytes of device
 * memory: kept positions int32 [num_seqs, budget], then context lengths int32
 * [num_seqs]; when max_blocks_per_seq * block_size exceeds 12288 tokens (the
 * selection is then split over 4096-token chunks, nch = ceil(max_ctx / 4096)
 * of them) also ranking keys uint32 [num_seqs, max_ctx rounded up to a
 * multiple of 4], per-chunk histograms uint32 [num_seqs, nch, 256], per-sequence histograms uint32 [num_seqs, 2,
 * 256], states int32 [3, num_seqs, 2] and per-chunk counts uint32 [num_seqs,
 * nch, 257]; each part rounded up to 256 bytes (0 for a NULL shape, a
 * negative num_seqs or a negative budget).  16-byte aligned, contents
 * irrelevant; no two calls may use it at once.  Two kernel launches, or seven
 * for the split selection (whose move is also split: first the kept tokens
 * whose source lies below the budget, in order, then all others at once).
 * Caller contract (not checked): valid and pairwise distinct block ids for
 * every logical block of every sequence with n > budget.
 */
size_t paged_kv_compress_workspace_bytes(const pa_score_shape *shape, int32_t budget);

int paged_kv_compress_prefill(void *k_cache, void *v_cache, float *scores,
                              const int32_t *block_tables, int32_t *context_lens, int32_t budget,
                              const pa_score_shape *shape, void *workspace, size_t workspace_bytes,
                              void *stream);

int paged_kv_compress_prefill_int8(int8_t *k_cache, int8_t *v_cache, float *k_scales,
                                   float *v_scales, float *scores, const int32_t *block_tables,
                                   int32_t *context_lens, int32_t budget,
                                   const pa_score_shape *shape, void *workspace,
                                   size_t workspace_bytes, void *stream);

int paged_kv_compress_prefill_fp8(uint8_t *k_cache, uint8_t *v_cache, float *scores,
                                  const int32_t *block_tables, int32_t *context_lens,
                                  int32_t budget, const pa_score_shape *shape, void *workspace,
                                  size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_EVICT_H */
