/*
 * paged_kv_write.h -- C-ABI of the KV write path of the MI355X (gfx950)
 * paged KV cache library: storing the new tokens' keys and values into the
 * paged cache that the paged_attn_decode entry points read (bf16, int8 or
 * FP8 E4M3).
 *
 * The operation: token t of the call owns the global token slot
 * slot_mapping[t], the address that BlockTable.append_slot hands out on the
 * ybb.press page "LLM 推理 KV Cache 内存管理深度工程实践：从 PageAttention
 * 到推测解码", section 2.1: block * block_size + offset.  Its key row for kv
 * head g is stored at k_cache[block, offset, g, :] and its value row at
 * v_cache[block, offset, g, :].  Because the cache layout is
 * [num_blocks, block_size, num_kv_heads, head_dim], that is row
 * slot * num_kv_heads + g of the cache seen as [num_blocks * block_size *
 * num_kv_heads, head_dim].  A negative slot (a token that received no slot,
 * e.g. padding) writes nothing.
 *
 * Layouts (row-major; all pointers are DEVICE memory owned by the caller):
 *   key, value      bf16 [num_tokens, num_kv_heads, head_dim]; consecutive
 *                   tokens are key_stride (value_stride) elements apart, so
 *                   K and V may be slices of a fused projection output
 *   slot_mapping    int32 [num_tokens]
 *   k_cache/v_cache bf16 (or int8) [num_blocks, block_size, num_kv_heads, head_dim]
 *   k_scales/v_scales fp32 [num_blocks, block_size, num_kv_heads]   (int8 only)
 * The per-layer slices of a layered cache are passed exactly as for decode.
 *
 * Ownership and state: the library allocates nothing and keeps no state.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *
 * Errors: PA_OK or a negative PA_ERR_* code of paged_attn.h, detected on the
 * host before any launch (nothing is written then).  Not checked (it would
 * need a device read): distinct non-negative slots -- two tokens given the
 * same slot race and either row may win.  Slots at or beyond
 * num_blocks * block_size are skipped by the kernel, never written.
 */
#ifndef PAGED_KV_WRITE_H
#define PAGED_KV_WRITE_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_write_shape {
    int32_t num_tokens;   /* T >= 0; T * num_kv_heads < 2^27.  T == 0 returns PA_OK
                             after the shape checks, without looking at the pointers */
    int32_t num_kv_heads; /* Hkv >= 1 */
    int32_t head_dim;     /* 64 or 128 */
    int32_t block_size;   /* tokens per block, >= 1 */
    int32_t num_blocks;   /* blocks in the pool, >= 1 */
    int32_t key_stride;   /* elements from token t's key row to token t+1's; 0 = Hkv*head_dim */
    int32_t value_stride; /* the same for value */
} pa_write_shape;

/*
 * bf16 cache: copies the rows unchanged.  key / value and both caches must be
 * 16-byte aligned and the strides multiples of 8 elements (PA_ERR_ALIGNMENT);
 * a stride below num_kv_heads * head_dim is PA_ERR_SHAPE.  One kernel launch.
 */
int paged_kv_write(const void *key, const void *value, const int32_t *slot_mapping,
                   void *k_cache, void *v_cache, const pa_write_shape *shape, void *stream);

/*
 * int8 cache: each (token, kv head) row x of head_dim values is quantized on
 * the way in with the symmetric recipe of the same page, section 6.1:
 * scale = max_i |x_i| / 127 in fp32, code_i = x_i / scale rounded half to
 * even and clamped to [-127, 127]; a row of zeros gets scale 0 and codes 0.
 * The codes go to k_cache / v_cache, the scale to k_scales / v_scales at the
 * same (block, offset, g).  key / value rows must hold finite values.  Same
 * alignment rules as paged_kv_write (the caches 8-byte aligned, the scale
 * arrays 4-byte aligned).  One kernel launch.
 */
int paged_kv_write_int8(const void *key, const void *value, const int32_t *slot_mapping,
                        int8_t *k_cache, int8_t *v_cache, float *k_scales, float *v_scales,
                        const pa_write_shape *shape, void *stream);

/*
 * FP8 E4M3 cache: each element is cast to its float8_e4m3fn code (the cast of
 * the same page, section 6.1, as torch performs it): round to nearest even,
 * subnormals kept, a magnitude past 464 (beyond the largest finite value 448),
 * an infinity or a NaN gives the NaN code with the value's sign (0x7F / 0xFF).
 * No scale.  k_cache / v_cache: uint8 codes [num_blocks, block_size,
 * num_kv_heads, head_dim], 8-byte aligned.  One kernel launch.
 */
int paged_kv_write_fp8(const void *key, const void *value, const int32_t *slot_mapping,
                       uint8_t *k_cache, uint8_t *v_cache, const pa_write_shape *shape,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_WRITE_H */
