/*
 * paged_attn.h -- C-ABI of the MI355X (gfx950) PagedAttention decode library.
 *
 * The operation (all entry points below compute it):
 *   For every sequence s and query head h, with G = num_q_heads / num_kv_heads
 *   and g = h / G, the single decode query q[s,h,:] attends over the
 *   context_lens[s] tokens of its sequence.  Token t lives in physical block
 *   block_tables[s][t / block_size], slot t % block_size.  Scores are
 *   scale * q . k_t; ONE softmax runs over all tokens of the sequence (not per
 *   block); out[s,h,:] = sum_t softmax_t * v_t.
 *   Passages: ybb.press page "LLM 推理 KV Cache 内存管理深度工程实践：从
 *   PageAttention 到推测解码", section 2.2 (block-table addressing, valid
 *   slots min(block_size, n - j*block_size), zero output for an empty context,
 *   q.K^T * scale) and section 6.2 (G consecutive query heads share one KV
 *   head); t6page "KV cache" page, section "PagedAttention 的算子" (contiguous
 *   K/V inside a block, softmax after merging all blocks).
 *
 * Layouts (all row-major, all pointers are DEVICE memory owned by the caller):
 *   q             bf16  [num_seqs, num_q_heads, head_dim]
 *   k_cache       bf16  [num_blocks, block_size, num_kv_heads, head_dim]
 *   v_cache       bf16  same layout as k_cache
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]
 *   context_lens  int32 [num_seqs]
 *   out           fp32  [num_seqs, num_q_heads, head_dim]
 *   The per-layer slices of a layered cache [2, L, num_blocks, block_size,
 *   num_kv_heads, head_dim] (nano-vLLM page, physical memory layout section)
 *   are passed as k_cache = base + (0*L + l)*slice, v_cache = base + (1*L + l)
 *   * slice; the library needs nothing else for that layout.
 *
 * Ownership and state: the library allocates nothing and keeps no per-call
 * state (paged_attn_decode_noalloc works in a static device array of the
 * library instead of a caller workspace; see there).  Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 * null stream) and stream-ordered with the caller's other work.
 *
 * Errors: every entry point returns PA_OK (0) or a negative PA_ERR_* code.
 * Argument errors are detected on the host before anything is launched, and
 * `out` is then left untouched.  Not checked (it would need a device read):
 * context_lens[s] <= max_blocks_per_seq * block_size and every table entry
 * j < ceil(context_lens[s] / block_size) in [0, num_blocks).  Entries at or
 * beyond that count, token slots at or beyond the context length and blocks
 * no table references are never read.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_OK 0
#define PA_ERR_NULL (-1)        /* a required pointer is NULL */
#define PA_ERR_SHAPE (-2)       /* non-positive size, q heads not a multiple of kv heads, ... */
#define PA_ERR_UNSUPPORTED (-3) /* head_dim or block_size with no compiled kernel */
#define PA_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than paged_attn_workspace_bytes */
#define PA_ERR_LAUNCH (-5)      /* the HIP runtime reported a launch error */
#define PA_ERR_ALIGNMENT (-6)   /* q, k_cache, v_cache, out or workspace not 16-byte aligned */
#define PA_ERR_SCRATCH (-7)     /* more scratch needed than paged_attn_decode_noalloc holds */

typedef struct pa_shape {
    int32_t num_seqs;           /* S  >= 0 (0 is a no-op) */
    int32_t num_q_heads;        /* Hq >= 1 */
    int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t head_dim;           /* 64 or 128 */
    int32_t block_size;         /* tokens per block: a power of two, 16 .. 4096 */
    int32_t max_blocks_per_seq; /* row length of block_tables, >= 1 */
    int32_t num_blocks;         /* blocks in the pool, >= 1 */
    int32_t split_tokens;       /* work item length in tokens (multiple of 16); 0 = balanced */
} pa_shape;

/*
 * How the work is split.  The contexts of all sequences, cut into 16-token
 * tiles, form one list; each workgroup of the (persistent) grid processes
 * "items" of that list.  With split_tokens == 0 the list is divided evenly
 * among the workgroups the device holds at once (at least 4 tiles per item);
 * otherwise items are split_tokens long.  A sequence that spans several items
 * is computed in parts whose (max, sum, weighted values) are merged with
 * log-sum-exp weights in a fixed order (the cross-split softmax reduction of a
 * split-context decode), so results are reproducible run to run.  Which
 * sequences are split depends only on the context lengths and the plan, never
 * on the block tables.
 * *split_tokens receives the item length (0 = balanced) and *max_splits the
 * largest number of items a call can use.  Returns PA_OK or an error.
 */
int paged_attn_plan(const pa_shape *shape, int32_t *split_tokens, int32_t *max_splits);

/*
 * Device workspace (bytes) a decode call with `shape` needs: partial results
 * fp32 [ceil(units/4), S + max_splits, 4, min(G, 16), head_dim + 2] (units =
 * Hkv * ceil(G / 16), G = Hq / Hkv), then int32 [S, 2] (the first and last
 * item holding each sequence), each part rounded up to 256 bytes.  It does
 * not depend on the device.  The contents need no initialisation; calls that
 * may run concurrently must not share a workspace.  Returns 0 on an invalid
 * shape; the decode call then reports the shape error.
 */
size_t paged_attn_workspace_bytes(const pa_shape *shape);

/*
 * bf16 KV cache decode.  `scale` is the softmax scale (1/sqrt(head_dim) for
 * standard attention).  `workspace` must hold paged_attn_workspace_bytes
 * bytes.  Two kernel launches on `stream`: the decode kernel, sized to the
 * current device, and the merge of the sequences it split.
 */
int paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      float *out, const pa_shape *shape, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * int8 KV cache decode: symmetric codes with one fp32 scale per (block,
 * slot, kv head) for K and for V separately, the dequantized value being
 * code * scale (ybb.press page, section 6.1, per-row amax/127 quantization).
 *   k_cache, v_cache    int8 [num_blocks, block_size, num_kv_heads, head_dim]
 *   k_scales, v_scales  fp32 [num_blocks, block_size, num_kv_heads]
 * Dequantization is fused into the kernel; everything else as
 * paged_attn_decode.
 */
int paged_attn_decode_int8(const void *q, const int8_t *k_cache, const int8_t *v_cache,
                           const float *k_scales, const float *v_scales,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           float *out, const pa_shape *shape, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * FP8 E4M3 KV cache: each element is a float8_e4m3fn code (OCP E4M3 "FN": 1
 * sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, NaN = codes
 * 0x7F / 0xFF, largest finite 448), the cast of the cache that the ybb.press
 * page, section 6.1, gives for inference; there is no scale.
 *   k_cache, v_cache  uint8 codes [num_blocks, block_size, num_kv_heads, head_dim]
 * Each code is decoded exactly (every E4M3 value is a bf16 value) inside the
 * kernel; everything else as paged_attn_decode.  A NaN code in a token the
 * context reads makes that sequence's output NaN, as the definition says.
 */
int paged_attn_decode_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                          const int32_t *block_tables, const int32_t *context_lens, float scale,
                          float *out, const pa_shape *shape, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Allocation-free bf16 decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, kernels and results (bit for bit) as
 * paged_attn_decode, with the partial results and item ranges in a static
 * device array of the library (32 MiB, held by each device the library runs
 * on until the process ends) instead of a caller workspace.  The caller still
 * passes the inputs and `out`; the call allocates nothing.
 * Scratch needed: ceil256(ceil(units/4) * (S + items) * 4 * min(G, 16) *
 * (head_dim + 2) * 4) + ceil256(8 * S) bytes, where items is the number of
 * workgroups of the decode grid (at most 512 on MI355X) with split_tokens == 0,
 * else the number of split_tokens items the table rows can hold.  A shape
 * needing more than 32 MiB is rejected with PA_ERR_SCRATCH before anything
 * is launched.  Nothing in the array needs clearing: a call writes every
 * entry it reads.  Every call on one device shares that device's array, so
 * calls that overlap on one device (other streams, other host threads) race:
 * the caller serialises them.
 */
int paged_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              float scale, float *out, const pa_shape *shape, void *stream);

/*
 * Device-side check of the caller contract that the decode (and the prefill,
 * scoring and compression) entry points do not check, since it needs a device
 * read: for every sequence s, 0 <= context_lens[s] <= max_blocks_per_seq *
 * block_size, and block_tables[s][j] lies in [0, num_blocks) for every
 * j < ceil(context_lens[s] / block_size).  It reads only block_tables and
 * context_lens (device memory), never a cache, so it is safe on arguments
 * that break the contract.  It writes, in device memory, result[0] = the
 * number of sequences that break it and result[1] = the lowest such s, or -1.
 * One kernel launch of one workgroup on `stream`; no workspace.  Meant for
 * debugging a caller: it does not change what the other entry points do.
 */
int paged_attn_check_tables(const int32_t *block_tables, const int32_t *context_lens,
                            int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                            int32_t num_blocks, int32_t *result, void *stream);

/* Static description of an error code; never NULL. */
const char *paged_attn_strerror(int code);

/* ABI version of this header (incremented on incompatible changes). */
int paged_attn_abi_version(void);

#define PA_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
