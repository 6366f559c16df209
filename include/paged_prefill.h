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
 * kernel launch (two for a key-split call, below), asynchronous on `stream` (a
 * hipStream_t; NULL = the null stream).  Errors: PA_OK or a negative PA_ERR_* code of paged_attn.h,
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
 * scores and the weighted values; accumulation is fp32.  V enters the second
 * product as fp16 (exact for every bf16 value below 2^16 in magnitude) and the
 * softmax weights as fp16 (2^-11 relative rounding; the row sums add the same
 * rounded weights).  A workgroup that meets a V value of magnitude 2^16 or
 * more (or an infinite one) computes its rows again with V as bf16 and the
 * weights as a bf16 high part plus remainder, so no V value is rounded.
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
 * paged_kv_write_int8.  The K codes enter the scores' product exactly (bf16)
 * and the K scales multiply the scores.  Each V scale s = m 2^e (mantissa m
 * in [1, 2)) is split: the V codes enter the weighted sum times 2^e, exactly,
 * as fp16; the weights enter as fp16 (2^-11 relative rounding) carrying m,
 * and the row sums add each rounded weight over m (an extra matrix product
 * with 1/m as an fp16 pair), so the rounding cancels in the quotient as on
 * the bf16 path.  A workgroup that meets a V scale outside 2^-14 .. 2^9
 * (other than 0: negative, tiny, huge or not finite) computes its rows again
 * with the weights times the whole V scales as a bf16 pair (exact to 2^-17);
 * so does every workgroup when |scale| log2(e) lies outside 2^-100 .. 2^100
 * (scale 0 included).
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

/*
 * Key-split prefill.  Each (sequence, kv head, tile of 256 query rows) is a
 * unit whose keys run over tiles of 32 tokens, from token 0 to its last row's
 * position.  With one workgroup per unit, a batch of few units (one 512-token
 * chunk of one sequence: 8 kv heads x 8 row tiles = 64 units) leaves most of
 * the GPU idle.  With key_splits = K > 1, the unit's key tiles are cut into
 * min(K, tiles) near-equal runs, one workgroup each.  Each run writes its rows'
 * unnormalised weighted sums, running maximum and row sum (fp32) to
 * `workspace`, and a second kernel combines the runs of each row: out =
 * sum_k e^(m_k - M) acc_k / sum_k e^(m_k - M) l_k (M the largest m_k): one
 * softmax over the row's whole visible context, as the unsplit call and the
 * decode's merge compute it (ybb.press page, section 2.2).  It differs from
 * the unsplit call's result by rounding only: fp32 summation order, and on
 * the bf16 and FP8 paths the fp16 weights rounded against each run's own
 * running maximum (within the same error bound; 1.2e-4 apart at most on a
 * 512-token Llama-3-8B chunk).  A unit with a single run writes out directly.
 *
 * paged_attn_prefill_plan: a key_splits for `shape` on the current device:
 * the smallest K for which the units' runs cover the compute units (one
 * prefill workgroup fills a compute unit), at most max_blocks_per_seq *
 * block_size / 128 (four or more tiles a run), at most 64; 1 when the units
 * already cover the GPU.  Units are counted from max_q_len, an upper bound.
 * Returns PA_OK, PA_ERR_NULL, a shape error as the prefill calls, or
 * PA_ERR_LAUNCH if the device cannot be queried.
 *
 * paged_attn_prefill_workspace_bytes: the workspace a key-split call with
 * `shape` and key_splits needs: num_seqs * Hkv * ceil(max_q_len * G / 256) *
 * key_splits * 256 rows of (head_dim + 2) floats; 0 when key_splits == 1 (no
 * workspace is read) or the shape or key_splits is invalid.
 *
 * paged_attn_prefill_split / _int8 / _fp8: the prefill calls above, with the
 * same arguments and per-run arithmetic, plus key_splits (1 .. 64; 1 is the unsplit
 * call and ignores the workspace) and a caller-owned device workspace
 * (16-byte aligned, at least paged_attn_prefill_workspace_bytes; contents
 * need no initialisation; calls that may run concurrently must not share
 * one).  Two kernel launches on `stream` when key_splits > 1.  Errors as the
 * unsplit calls, plus PA_ERR_SHAPE for key_splits outside 1 .. 64,
 * PA_ERR_WORKSPACE for a NULL or too small workspace and PA_ERR_ALIGNMENT
 * for a misaligned one, all before any launch.
 */
int paged_attn_prefill_plan(const pa_prefill_shape *shape, int32_t *key_splits);

size_t paged_attn_prefill_workspace_bytes(const pa_prefill_shape *shape, int32_t key_splits);

int paged_attn_prefill_split(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, const int32_t *context_lens,
                             const int32_t *q_offsets, float scale, float *out,
                             const pa_prefill_shape *shape, int32_t key_splits, void *workspace,
                             size_t workspace_bytes, void *stream);

int paged_attn_prefill_split_int8(const void *q, const int8_t *k_cache, const int8_t *v_cache,
                                  const float *k_scales, const float *v_scales,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *q_offsets, float scale, float *out,
                                  const pa_prefill_shape *shape, int32_t key_splits,
                                  void *workspace, size_t workspace_bytes, void *stream);

int paged_attn_prefill_split_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *q_offsets, float scale, float *out,
                                 const pa_prefill_shape *shape, int32_t key_splits,
                                 void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_PREFILL_H */
