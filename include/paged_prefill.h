/*
 * paged_prefill.h -- C-ABI of paged chunked-prefill attention in the MI355X
 * (gfx950) paged KV cache library.
 *
 * The operation (ybb.press page "LLM 推理 KV Cache 内存管理深度工程实践", section
 * 7.3: a long prompt's prefill is cut into 512-token chunks run between the
 * decodes; t6page "KV cache" page, section "Chunked prefill：让 prefill 不阻塞
 * decode": one batch = one prefill chunk + all decodes).  Every sequence s
 * brings n_q[s] = q_offsets[s+1] - q_offsets[s] query tokens: the LAST n_q[s]
 * tokens of its context, whose K/V are already in the paged cache (written
 * with paged_kv_write).  Query i of s is at position
 * p = context_lens[s] - n_q[s] + i and attends causally to tokens 0 .. p of
 * its sequence through the block table, with the decode definition: scores
 * scale * q.k, one softmax, weighted V, G = Hq/Hkv consecutive query heads per
 * kv head.  n_q = 1 is a decode, so one call can carry a prefill chunk and
 * decodes together.
 *
 * Layouts (row-major; all pointers are DEVICE memory owned by the caller):
 *   q             bf16 [q_offsets[S], Hq, head_dim]  (sequence s: rows q_offsets[s] ..)
 *   k_cache, v_cache  bf16 [num_blocks, block_size, Hkv, head_dim]
 *   block_tables  int32 [S, max_blocks_per_seq];  context_lens int32 [S]
 *   q_offsets     int32 [S + 1], q_offsets[0] = 0, non-decreasing
 *   out           fp32 [q_offsets[S], Hq, head_dim]
 *
 * Ownership and state: the library allocates nothing and keeps no state; one
 * kernel launch, asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream).  Errors: PA_OK or a negative PA_ERR_* code of paged_attn.h,
 * detected on the host before the launch (out untouched then).  Not checked
 * (device data): n_q[s] <= max_q_len, n_q[s] <= context_lens[s] <=
 * max_blocks_per_seq * block_size, valid block ids for every block a context
 * uses.  Slots past each context end are never read.
 */
#ifndef PAGED_PREFILL_H
#define PAGED_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_prefill_shape {
    int32_t num_seqs;           /* S >= 0 (0 is a no-op) */
    int32_t num_q_heads;        /* Hq >= 1, a multiple of Hkv */
    int32_t num_kv_heads;       /* Hkv >= 1 */
    int32_t head_dim;           /* 64 or 128 */
    int32_t block_size;         /* a power of two, 16 .. 4096 */
    int32_t max_blocks_per_seq; /* >= 1 */
    int32_t num_blocks;         /* >= 1 */
    int32_t max_q_len;          /* >= 1: no sequence brings more query tokens */
} pa_prefill_shape;

/*
 * Chunked-prefill attention over a bf16 cache.  Matrix cores compute the
 * scores and the weighted values; the softmax weights enter the second product
 * as a bf16 high part plus a bf16 remainder (exact to 2^-17 relative);
 * accumulation is fp32.
 */
int paged_attn_prefill(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens,
                       const int32_t *q_offsets, float scale, float *out,
                       const pa_prefill_shape *shape, void *stream);

/*
 * The same chunked prefill over an int8 cache (ybb.press page, section 6.1:
 * element = code * scale): k_cache / v_cache int8 codes [num_blocks,
 * block_size, Hkv, head_dim] (8-byte aligned), k_scales / v_scales fp32
 * [num_blocks, block_size, Hkv] (4-byte aligned), as written by
 * paged_kv_write_int8.  The codes enter the matrix products exactly (bf16);
 * the K scales multiply the scores, the V scales the weights.
 */
int paged_attn_prefill_int8(const void *q, const int8_t *k_cache, const int8_t *v_cache,
                            const float *k_scales, const float *v_scales,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const int32_t *q_offsets, float scale, float *out,
                            const pa_prefill_shape *shape, void *stream);

/*
 * The same chunked prefill over an FP8 E4M3 cache (uint8 codes, OCP E4M3 as
 * torch's float8_e4m3fn, 8-byte aligned), as written by paged_kv_write_fp8.
 * Every code's value is exact in bf16 (K) and fp16 (V).  The weights enter
 * the second product as fp16 (2^-11 relative rounding, the row sums adding
 * the same rounded weights), one product instead of two: within the 2e-3
 * absolute bar with a margin (about 4e-4 measured at 4096 tokens), not
 * exact to 2^-17 as on the bf16 and int8 paths.
 */
int paged_attn_prefill_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           const int32_t *q_offsets, float scale, float *out,
                           const pa_prefill_shape *shape, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_PREFILL_H */
