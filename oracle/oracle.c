/*
 * oracle.c -- plain, slow, fp64 CPU reference for PagedAttention decode, for
 * the KV write path that fills the paged cache, and for PagedEviction's token
 * importance and block eviction (the last two at the end of this file).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's cpu_baseline leg may load this library.  It shares no code, header,
 * table or helper with the HIP library; it is compiled with gcc on its own.
 *
 * What it computes (the plain definition, no blocking, no online softmax, no
 * splits):
 *
 *   For every sequence s and query head h, with G = Hq / Hkv, g = h / G and
 *   n = context_lens[s]:
 *     - n == 0            -> out[s,h,:] = 0
 *     - token t in [0,n)  -> physical block b = block_tables[s][t / BS],
 *                            slot r = t % BS, key k_t = K[b, r, g, :],
 *                            value v_t = V[b, r, g, :]
 *     - score             s_t = scale * sum_i q[s,h,i] * k_t[i]
 *     - softmax over ALL n tokens of the sequence (two passes: max, then
 *       exp/sum), out[s,h,:] = sum_t e_t v_t / sum_t e_t.
 *
 * Passages followed:
 *   - page "LLM 推理 KV Cache 内存管理深度工程实践：从 PageAttention 到推测解码"
 *     (ybb.press), section 2.2 (paged attention): the logical block index
 *     maps through the block table to a physical block, a block holds
 *     block_size token slots, only min(block_size, n - j*block_size) slots of
 *     block j are valid, the output starts at zero, scores are q.K^T * scale.
 *     Its per-block softmax is read as ONE softmax over the whole context, as
 *     the next passage states.
 *   - page "KV cache" (t6page.pages.dev), section "PagedAttention 的算子":
 *     K/V are contiguous inside a block, and the scaled dot product and the
 *     softmax are taken after all blocks are merged.
 *   - same ybb.press page, section 6.2 (GQA/MQA cache sharing): each group of
 *     G consecutive query heads shares one KV head (read as g = h / G).
 *   - same ybb.press page, section 6.1 (INT8 KV): symmetric quantization with
 *     scale = amax(|x|) / 127 over the head dimension; the int8 entry point
 *     dequantizes k_t = code * scale before the definition above.  The same
 *     section casts the cache to FP8 E4M3 (float8_e4m3fn) with no scale; the
 *     fp8 entry point decodes each code exactly before the definition above.
 *
 * Precision: every input is widened exactly to double (bf16 -> double and
 * int8 -> double are exact; the fp32 scale is taken as double(scale_f32)).
 * The caller contract (valid block ids for every logical block below
 * ceil(n/BS)) is CHECKED here: the oracle returns a negative code instead of
 * reading out of bounds.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_TABLE (-2)
#define ORC_ERR_NOMEM (-3)

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Element kinds of the KV cache. */
enum { KV_BF16 = 0, KV_INT8 = 1, KV_FP8 = 2 };

/*
 * FP8 E4M3 (the OCP "FN" variant that torch.float8_e4m3fn names; the ybb.press
 * page, section 6.1, casts the cache to it for inference): 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits, no infinities, and NaN only for
 * exponent and mantissa all ones (codes 0x7F and 0xFF).  Exponent field 0 holds
 * the subnormals m * 2^-9.  Decoded exactly to double.
 */
double oracle_fp8_e4m3_to_double(uint8_t code)
{
    const int sign = code >> 7;
    const int e = (code >> 3) & 15;
    const int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/*
 * The code of x after the cast to E4M3: the nearest finite E4M3 value, ties
 * to the even code (mantissa LSB 0).  A magnitude that rounds past the largest
 * finite value 448 (i.e. above the midpoint 464 between 448 and the next step
 * 480, which is the NaN pattern), an infinity and a NaN give the NaN code with
 * x's sign -- the conversion torch's cast performs.  Found by comparing x with
 * every finite code, so no bit tricks are involved.
 */
uint8_t oracle_fp8_e4m3_from_double(double x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x) || isinf(x)) return (uint8_t)(sign | 0x7F);
    const double a = fabs(x);
    if (a > 464.0) return (uint8_t)(sign | 0x7F);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {            /* non-negative finite codes */
        const double d = fabs(oracle_fp8_e4m3_to_double((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* Array forms of the two conversions above (for the tests). */
void oracle_fp8_e4m3_decode_array(const uint8_t *codes, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_e4m3_to_double(codes[i]);
}

void oracle_fp8_e4m3_encode_array(const double *x, int64_t n, uint8_t *codes)
{
    for (int64_t i = 0; i < n; ++i) codes[i] = oracle_fp8_e4m3_from_double(x[i]);
}

typedef struct {
    int kind;
    const void *k;          /* [NB, BS, Hkv, D] bf16 bits, int8 codes or fp8 codes */
    const void *v;
    const float *k_scales;  /* [NB, BS, Hkv], int8 only */
    const float *v_scales;
} kv_src;

/* Key or value element i of token slot (b, r) for kv head g, widened to double. */
static double kv_elem(const kv_src *src, int which_v, int64_t b, int r, int g, int i,
                      int BS, int Hkv, int D)
{
    int64_t slot = (b * BS + r) * (int64_t)Hkv + g;
    if (src->kind == KV_BF16) {
        const uint16_t *base = (const uint16_t *)(which_v ? src->v : src->k);
        return bf16_bits_to_double(base[slot * D + i]);
    } else if (src->kind == KV_FP8) {
        const uint8_t *base = (const uint8_t *)(which_v ? src->v : src->k);
        return oracle_fp8_e4m3_to_double(base[slot * D + i]);
    } else {
        const int8_t *base = (const int8_t *)(which_v ? src->v : src->k);
        const float *sc = which_v ? src->v_scales : src->k_scales;
        return (double)base[slot * D + i] * (double)sc[slot];
    }
}

static int decode_common(const uint16_t *q, const kv_src *src,
                         const int32_t *block_tables, const int32_t *context_lens,
                         int S, int Hq, int Hkv, int D, int BS, int MB, int64_t NB,
                         float scale, double *out)
{
    if (!q || !src->k || !src->v || !block_tables || !context_lens || !out) return ORC_ERR_ARG;
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || MB < 0 || NB < 0) return ORC_ERR_ARG;
    if (Hq % Hkv != 0) return ORC_ERR_ARG;
    if (src->kind == KV_INT8 && (!src->k_scales || !src->v_scales)) return ORC_ERR_ARG;

    /* Check the caller contract before any gather. */
    for (int s = 0; s < S; ++s) {
        int n = context_lens[s];
        if (n < 0 || (int64_t)n > (int64_t)MB * BS) return ORC_ERR_TABLE;
        int nblk = (n + BS - 1) / BS;
        for (int j = 0; j < nblk; ++j) {
            int32_t b = block_tables[(int64_t)s * MB + j];
            if (b < 0 || (int64_t)b >= NB) return ORC_ERR_TABLE;
        }
    }

    const int G = Hq / Hkv;
    const double sc = (double)scale;
    int err = ORC_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < (int64_t)S * Hq; ++row) {
        const int s = (int)(row / Hq);
        const int h = (int)(row % Hq);
        const int g = h / G;
        const int n = context_lens[s];
        double *o = out + row * D;
        for (int i = 0; i < D; ++i) o[i] = 0.0;
        if (n == 0) continue;

        double *scores = (double *)malloc(sizeof(double) * (size_t)n);
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!scores || !qd) {
            free(scores);
            free(qd);
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
            continue;
        }
        for (int i = 0; i < D; ++i) qd[i] = bf16_bits_to_double(q[row * D + i]);

        /* Pass 1: scores over the gathered context, and their maximum. */
        double m = -INFINITY;
        for (int t = 0; t < n; ++t) {
            int64_t b = block_tables[(int64_t)s * MB + t / BS];
            int r = t % BS;
            double dot = 0.0;
            for (int i = 0; i < D; ++i) dot += qd[i] * kv_elem(src, 0, b, r, g, i, BS, Hkv, D);
            scores[t] = sc * dot;
            if (scores[t] > m) m = scores[t];
        }
        /* Pass 2: exponentials, their sum, and the weighted sum of values. */
        double denom = 0.0;
        for (int t = 0; t < n; ++t) {
            int64_t b = block_tables[(int64_t)s * MB + t / BS];
            int r = t % BS;
            double e = exp(scores[t] - m);
            denom += e;
            for (int i = 0; i < D; ++i) o[i] += e * kv_elem(src, 1, b, r, g, i, BS, Hkv, D);
        }
        for (int i = 0; i < D; ++i) o[i] /= denom;
        free(scores);
        free(qd);
    }
    return err;
}

/*
 * bf16 KV cache.  q: bf16 bits [S, Hq, D]; k_cache / v_cache: bf16 bits
 * [NB, BS, Hkv, D]; block_tables: int32 [S, MB]; context_lens: int32 [S];
 * out: double [S, Hq, D].  Returns 0, or a negative code.
 */
int oracle_paged_decode_bf16(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                             const int32_t *block_tables, const int32_t *context_lens,
                             int S, int Hq, int Hkv, int D, int BS, int MB, int64_t NB,
                             float scale, double *out)
{
    kv_src src = {KV_BF16, k_cache, v_cache, NULL, NULL};
    return decode_common(q, &src, block_tables, context_lens, S, Hq, Hkv, D, BS, MB, NB, scale, out);
}

/*
 * int8 KV cache with one fp32 scale per (token slot, kv head), for K and V
 * separately.  k_cache / v_cache: int8 [NB, BS, Hkv, D]; k_scales /
 * v_scales: fp32 [NB, BS, Hkv].  The rest as in the bf16 entry point.
 */
int oracle_paged_decode_int8(const uint16_t *q, const int8_t *k_cache, const int8_t *v_cache,
                             const float *k_scales, const float *v_scales,
                             const int32_t *block_tables, const int32_t *context_lens,
                             int S, int Hq, int Hkv, int D, int BS, int MB, int64_t NB,
                             float scale, double *out)
{
    kv_src src = {KV_INT8, k_cache, v_cache, k_scales, v_scales};
    return decode_common(q, &src, block_tables, context_lens, S, Hq, Hkv, D, BS, MB, NB, scale, out);
}

/*
 * FP8 E4M3 KV cache (ybb.press page, section 6.1: the cache cast to
 * float8_e4m3fn, no scale): k_cache / v_cache hold codes [NB, BS, Hkv, D],
 * each decoded exactly by oracle_fp8_e4m3_to_double.  The rest as in the bf16
 * entry point.
 */
int oracle_paged_decode_fp8(const uint16_t *q, const uint8_t *k_cache, const uint8_t *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int S, int Hq, int Hkv, int D, int BS, int MB, int64_t NB,
                            float scale, double *out)
{
    kv_src src = {KV_FP8, k_cache, v_cache, NULL, NULL};
    return decode_common(q, &src, block_tables, context_lens, S, Hq, Hkv, D, BS, MB, NB, scale, out);
}

/*
 * Symmetric per-row int8 quantizer, in fp32 as the page's tensor code does it
 * (page "LLM 推理 KV Cache 内存管理深度工程实践", section 6.1): the row's scale
 * is amax(|x|)/127 and each code is x/scale rounded half-to-even.  A row of
 * zeros gets scale 0 and codes 0 (the page's formula would divide by zero).
 * x: fp32 [rows, D]; codes: int8 [rows, D]; scales: fp32 [rows].
 */
void oracle_quantize_int8_rows(const float *x, int64_t rows, int D, int8_t *codes, float *scales)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * D;
        float amax = 0.0f;
        for (int i = 0; i < D; ++i) {
            float a = fabsf(xr[i]);
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        scales[r] = s;
        for (int i = 0; i < D; ++i) {
            float c = (s == 0.0f) ? 0.0f : nearbyintf(xr[i] / s);
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
            codes[r * D + i] = (int8_t)c;
        }
    }
}

/*
 * KV write path: each new token's key and value rows are stored at the token
 * slot the block table handed out for it.  The ybb.press page, section 2.1
 * (BlockTable.append_slot), gives a token's global slot address as
 * block * BS + offset (offset = slots already used in that block); the cache
 * position is therefore block = slot / BS, offset = slot % BS, and token t's
 * row for kv head g lands at cache[block, offset, g, :], in K and in V alike.
 * A negative slot marks a token with no slot (append_slot returned None, or a
 * padding token): nothing is written for it.
 *
 * key / value: bf16 bits; token t's row for kv head g starts at element
 * t * key_stride + g * D (resp. value_stride).  slots: int32 [T].
 * Checked before anything is written: every slot < NB * BS, and no slot
 * appears twice (two tokens cannot own one slot).  Returns 0 or a negative
 * code (the caches are then untouched).
 */
static int check_slots(const int32_t *slots, int T, int BS, int64_t NB)
{
    const int64_t n_slots = NB * (int64_t)BS;
    int64_t n_valid = 0;
    for (int t = 0; t < T; ++t) {
        if (slots[t] >= 0 && (int64_t)slots[t] >= n_slots) return ORC_ERR_TABLE;
        if (slots[t] >= 0) ++n_valid;
    }
    if (n_valid == 0) return ORC_OK;
    unsigned char *seen = (unsigned char *)calloc((size_t)n_slots, 1);
    if (!seen) return ORC_ERR_NOMEM;
    int rc = ORC_OK;
    for (int t = 0; t < T && rc == ORC_OK; ++t) {
        if (slots[t] < 0) continue;
        if (seen[slots[t]]) rc = ORC_ERR_ARG;
        seen[slots[t]] = 1;
    }
    free(seen);
    return rc;
}

int oracle_kv_write_bf16(const uint16_t *key, const uint16_t *value, const int32_t *slots,
                         int T, int Hkv, int D, int64_t key_stride, int64_t value_stride,
                         uint16_t *k_cache, uint16_t *v_cache, int BS, int64_t NB)
{
    if (T < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB < 0) return ORC_ERR_ARG;
    if (T > 0 && (!key || !value || !slots || !k_cache || !v_cache)) return ORC_ERR_ARG;
    int rc = check_slots(slots, T, BS, NB);
    if (rc != ORC_OK) return rc;
    for (int t = 0; t < T; ++t) {
        if (slots[t] < 0) continue;
        const int64_t block = slots[t] / BS;
        const int64_t offset = slots[t] % BS;
        for (int g = 0; g < Hkv; ++g) {
            const int64_t dst = ((block * BS + offset) * Hkv + g) * (int64_t)D;
            for (int i = 0; i < D; ++i) {
                k_cache[dst + i] = key[t * key_stride + (int64_t)g * D + i];
                v_cache[dst + i] = value[t * value_stride + (int64_t)g * D + i];
            }
        }
    }
    return ORC_OK;
}

/*
 * int8 KV write path: as oracle_kv_write_bf16, but each (token, kv head) row
 * is quantized on the way in with the section 6.1 recipe of the same page
 * (oracle_quantize_int8_rows on the row widened exactly from bf16 to fp32);
 * the codes go to the int8 caches [NB, BS, Hkv, D] and the row's scale to
 * k_scales / v_scales [NB, BS, Hkv] at the same (block, offset, g).
 */
int oracle_kv_write_int8(const uint16_t *key, const uint16_t *value, const int32_t *slots,
                         int T, int Hkv, int D, int64_t key_stride, int64_t value_stride,
                         int8_t *k_cache, int8_t *v_cache, float *k_scales, float *v_scales,
                         int BS, int64_t NB)
{
    if (T < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB < 0) return ORC_ERR_ARG;
    if (T > 0 && (!key || !value || !slots || !k_cache || !v_cache || !k_scales || !v_scales))
        return ORC_ERR_ARG;
    int rc = check_slots(slots, T, BS, NB);
    if (rc != ORC_OK) return rc;
    float *row = (float *)malloc(sizeof(float) * (size_t)D);
    if (!row) return ORC_ERR_NOMEM;
    for (int t = 0; t < T; ++t) {
        if (slots[t] < 0) continue;
        const int64_t block = slots[t] / BS;
        const int64_t offset = slots[t] % BS;
        for (int g = 0; g < Hkv; ++g) {
            const int64_t cell = (block * BS + offset) * Hkv + g;
            for (int i = 0; i < D; ++i)
                row[i] = (float)bf16_bits_to_double(key[t * key_stride + (int64_t)g * D + i]);
            oracle_quantize_int8_rows(row, 1, D, k_cache + cell * D, k_scales + cell);
            for (int i = 0; i < D; ++i)
                row[i] = (float)bf16_bits_to_double(value[t * value_stride + (int64_t)g * D + i]);
            oracle_quantize_int8_rows(row, 1, D, v_cache + cell * D, v_scales + cell);
        }
    }
    free(row);
    return ORC_OK;
}

/*
 * FP8 KV write path: as oracle_kv_write_bf16, each element of the token's
 * bf16 K / V rows cast to its E4M3 code (oracle_fp8_e4m3_from_double; the
 * bf16 value widens exactly) and stored at the same cache position.
 */
int oracle_kv_write_fp8(const uint16_t *key, const uint16_t *value, const int32_t *slots,
                        int T, int Hkv, int D, int64_t key_stride, int64_t value_stride,
                        uint8_t *k_cache, uint8_t *v_cache, int BS, int64_t NB)
{
    if (T < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB < 0) return ORC_ERR_ARG;
    if (T > 0 && (!key || !value || !slots || !k_cache || !v_cache)) return ORC_ERR_ARG;
    int rc = check_slots(slots, T, BS, NB);
    if (rc != ORC_OK) return rc;
    for (int t = 0; t < T; ++t) {
        if (slots[t] < 0) continue;
        const int64_t block = slots[t] / BS;
        const int64_t offset = slots[t] % BS;
        for (int g = 0; g < Hkv; ++g) {
            const int64_t dst = ((block * BS + offset) * Hkv + g) * (int64_t)D;
            for (int i = 0; i < D; ++i) {
                k_cache[dst + i] = oracle_fp8_e4m3_from_double(
                    bf16_bits_to_double(key[t * key_stride + (int64_t)g * D + i]));
                v_cache[dst + i] = oracle_fp8_e4m3_from_double(
                    bf16_bits_to_double(value[t * value_stride + (int64_t)g * D + i]));
            }
        }
    }
    return ORC_OK;
}

/*
 * PagedEviction, token importance (page "KV缓存内存布局优化：分页策略、量化压缩
 * 与动态驱逐的工程实践", section "PagedEviction 块级驱逐机制"): a token's
 * importance is the ratio of the L2 norms of its value and key,
 * S_t = ||V_t||_2 / ||K_t||_2, where K_t and V_t are the token's whole rows in
 * the layer's cache (all kv heads, all dims), dequantized like the decode
 * entry points.  The score is kept with the token's slot, like its K/V:
 * scores[b * BS + r] for the token in physical block b, slot r.  For every
 * sequence s, tokens t in [token_begin[s], context_lens[s]) (token_begin
 * NULL: from 0) are scored; other entries are left alone.  Norms and ratio in
 * double.
 */
static int token_scores_common(const kv_src *src, const int32_t *block_tables,
                               const int32_t *token_begin, const int32_t *context_lens,
                               int S, int Hkv, int D, int BS, int MB, int64_t NB, double *scores)
{
    if (!src->k || !src->v || !block_tables || !context_lens || !scores) return ORC_ERR_ARG;
    if (S < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || MB < 0 || NB < 0) return ORC_ERR_ARG;
    if (src->kind == KV_INT8 && (!src->k_scales || !src->v_scales)) return ORC_ERR_ARG;
    for (int s = 0; s < S; ++s) {
        int n = context_lens[s];
        int b0 = token_begin ? token_begin[s] : 0;
        if (n < 0 || (int64_t)n > (int64_t)MB * BS) return ORC_ERR_TABLE;
        if (b0 < 0) return ORC_ERR_ARG;
        int nblk = (n + BS - 1) / BS;
        for (int j = 0; j < nblk; ++j) {
            int32_t b = block_tables[(int64_t)s * MB + j];
            if (b < 0 || (int64_t)b >= NB) return ORC_ERR_TABLE;
        }
    }
    for (int s = 0; s < S; ++s) {
        const int n = context_lens[s];
        for (int t = token_begin ? token_begin[s] : 0; t < n; ++t) {
            const int64_t b = block_tables[(int64_t)s * MB + t / BS];
            const int r = t % BS;
            double kk = 0.0, vv = 0.0;
            for (int g = 0; g < Hkv; ++g) {
                for (int i = 0; i < D; ++i) {
                    const double kx = kv_elem(src, 0, b, r, g, i, BS, Hkv, D);
                    const double vx = kv_elem(src, 1, b, r, g, i, BS, Hkv, D);
                    kk += kx * kx;
                    vv += vx * vx;
                }
            }
            scores[b * BS + r] = sqrt(vv) / sqrt(kk);
        }
    }
    return ORC_OK;
}

int oracle_token_scores_bf16(const uint16_t *k_cache, const uint16_t *v_cache,
                             const int32_t *block_tables, const int32_t *token_begin,
                             const int32_t *context_lens, int S, int Hkv, int D, int BS, int MB,
                             int64_t NB, double *scores)
{
    kv_src src = {KV_BF16, k_cache, v_cache, NULL, NULL};
    return token_scores_common(&src, block_tables, token_begin, context_lens, S, Hkv, D, BS, MB,
                               NB, scores);
}

int oracle_token_scores_int8(const int8_t *k_cache, const int8_t *v_cache, const float *k_scales,
                             const float *v_scales, const int32_t *block_tables,
                             const int32_t *token_begin, const int32_t *context_lens, int S,
                             int Hkv, int D, int BS, int MB, int64_t NB, double *scores)
{
    kv_src src = {KV_INT8, k_cache, v_cache, k_scales, v_scales};
    return token_scores_common(&src, block_tables, token_begin, context_lens, S, Hkv, D, BS, MB,
                               NB, scores);
}

int oracle_token_scores_fp8(const uint8_t *k_cache, const uint8_t *v_cache,
                            const int32_t *block_tables, const int32_t *token_begin,
                            const int32_t *context_lens, int S, int Hkv, int D, int BS, int MB,
                            int64_t NB, double *scores)
{
    kv_src src = {KV_FP8, k_cache, v_cache, NULL, NULL};
    return token_scores_common(&src, block_tables, token_begin, context_lens, S, Hkv, D, BS, MB,
                               NB, scores);
}

/*
 * PagedEviction, decode-phase block eviction (same page and section: when
 * the newest block fills, the mean importance of every existing full block is
 * evaluated and the full block with the lowest mean is evicted whole).
 *
 * For each sequence s with evict_mask[s] != 0 and at least one full block
 * (n_full = context_lens[s] / BS):
 *   - the mean of full block j (physical block b = block_tables[s][j]) is
 *     (sum of its BS slot scores scores[b * BS + r], added in slot order in
 *     double) / BS, from the fp32 scores given (the importances the caller
 *     holds, so that both sides take the decision from the same bits);
 *   - the victim is the block with the smallest mean, the lowest j among
 *     equal means; NaN means are never chosen unless every mean is NaN (then
 *     block 0);
 *   - the victim leaves the table: entries j+1 .. nblk-1 move down by one and
 *     entry nblk-1 becomes -1; context_lens[s] -= BS; evicted[s] = the
 *     victim's physical block (free for reuse; its scores stay with it).
 * Otherwise evicted[s] = -1 and nothing changes.  Tables and lengths are
 * updated in place.
 */
int oracle_evict_lowest_block(const float *scores, int32_t *block_tables, int32_t *context_lens,
                              const int32_t *evict_mask, int32_t *evicted, int S, int MB, int BS,
                              int64_t NB)
{
    if (!scores || !block_tables || !context_lens || !evict_mask || !evicted) return ORC_ERR_ARG;
    if (S < 0 || MB <= 0 || BS <= 0 || NB < 0) return ORC_ERR_ARG;
    for (int s = 0; s < S; ++s) {
        const int n = context_lens[s];
        if (n < 0 || (int64_t)n > (int64_t)MB * BS) return ORC_ERR_TABLE;
        if (!evict_mask[s]) continue;
        for (int j = 0; j < (n + BS - 1) / BS; ++j) {
            int32_t b = block_tables[(int64_t)s * MB + j];
            if (b < 0 || (int64_t)b >= NB) return ORC_ERR_TABLE;
        }
    }
    for (int s = 0; s < S; ++s) {
        evicted[s] = -1;
        const int n = context_lens[s];
        const int n_full = n / BS;
        if (!evict_mask[s] || n_full == 0) continue;
        int32_t *row = block_tables + (int64_t)s * MB;
        int victim = -1;
        double best = 0.0;
        for (int j = 0; j < n_full; ++j) {
            const float *blk = scores + (int64_t)row[j] * BS;
            double sum = 0.0;
            for (int r = 0; r < BS; ++r) sum += (double)blk[r];
            const double mean = sum / BS;
            if (isnan(mean)) continue;
            if (victim < 0 || mean < best) {
                victim = j;
                best = mean;
            }
        }
        if (victim < 0) victim = 0;
        const int nblk = (n + BS - 1) / BS;
        evicted[s] = row[victim];
        for (int j = victim; j + 1 < nblk; ++j) row[j] = row[j + 1];
        row[nblk - 1] = -1;
        context_lens[s] = n - BS;
    }
    return ORC_OK;
}

/*
 * Paged chunked-prefill attention (ybb.press page, section 7.3: a long prompt's
 * prefill is cut into 512-token chunks that run alongside the decodes; the t6page
 * "KV cache" page, section "Chunked prefill：让 prefill 不阻塞 decode": one batch =
 * one prefill chunk + all decodes).  Every sequence s brings n_q = q_offsets[s+1] - q_offsets[s]
 * query tokens: the LAST n_q tokens of its context (their K/V already stored,
 * n_q <= context_lens[s]).  Query i of s sits at position
 * p = context_lens[s] - n_q + i and attends causally: to tokens 0 .. p of its
 * sequence, through the block table, with the decode definition (scores
 * scale * q.k, one softmax, weighted V; GQA g = h / G).  n_q = 1 is a decode.
 * q: bf16 [q_offsets[S], Hq, D]; out: double [q_offsets[S], Hq, D].
 */
static void attend_prefix(const double *qd, const kv_src *src, const int32_t *table_row, int n,
                          int g, int Hkv, int D, int BS, double sc, double *scores, double *o)
{
    for (int i = 0; i < D; ++i) o[i] = 0.0;
    if (n == 0) return;
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        const int64_t b = table_row[t / BS];
        const int r = t % BS;
        double dot = 0.0;
        for (int i = 0; i < D; ++i) dot += qd[i] * kv_elem(src, 0, b, r, g, i, BS, Hkv, D);
        scores[t] = sc * dot;
        if (scores[t] > m) m = scores[t];
    }
    double denom = 0.0;
    for (int t = 0; t < n; ++t) {
        const int64_t b = table_row[t / BS];
        const int r = t % BS;
        const double e = exp(scores[t] - m);
        denom += e;
        for (int i = 0; i < D; ++i) o[i] += e * kv_elem(src, 1, b, r, g, i, BS, Hkv, D);
    }
    for (int i = 0; i < D; ++i) o[i] /= denom;
}

static int prefill_common(const uint16_t *q, const kv_src *src, const int32_t *block_tables,
                          const int32_t *context_lens, const int32_t *q_offsets, int S, int Hq,
                          int Hkv, int D, int BS, int MB, int64_t NB, float scale, double *out)
{
    if (!q || !src->k || !src->v || !block_tables || !context_lens || !q_offsets || !out)
        return ORC_ERR_ARG;
    if (src->kind == KV_INT8 && (!src->k_scales || !src->v_scales)) return ORC_ERR_ARG;
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || MB < 0 || NB < 0 || Hq % Hkv)
        return ORC_ERR_ARG;
    if (q_offsets[0] != 0) return ORC_ERR_ARG;
    for (int s = 0; s < S; ++s) {
        const int n = context_lens[s];
        const int nq = q_offsets[s + 1] - q_offsets[s];
        if (nq < 0 || nq > n) return ORC_ERR_ARG;
        if (n < 0 || (int64_t)n > (int64_t)MB * BS) return ORC_ERR_TABLE;
        for (int j = 0; j < (n + BS - 1) / BS; ++j) {
            int32_t b = block_tables[(int64_t)s * MB + j];
            if (b < 0 || (int64_t)b >= NB) return ORC_ERR_TABLE;
        }
    }
    const int G = Hq / Hkv;
    const int64_t rows = (int64_t)q_offsets[S] * Hq;
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t row = 0; row < rows; ++row) {
        const int64_t qi = row / Hq;          /* query token index over the batch */
        const int h = (int)(row % Hq);
        int s = 0;
        while (q_offsets[s + 1] <= qi) ++s;
        const int nq = q_offsets[s + 1] - q_offsets[s];
        const int i = (int)(qi - q_offsets[s]);
        const int p = context_lens[s] - nq + i;            /* the query's position */
        double *scores = (double *)malloc(sizeof(double) * (size_t)(p + 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!scores || !qd) {
            free(scores);
            free(qd);
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
            continue;
        }
        for (int x = 0; x < D; ++x) qd[x] = bf16_bits_to_double(q[row * D + x]);
        attend_prefix(qd, src, block_tables + (int64_t)s * MB, p + 1, h / G, Hkv, D, BS,
                      (double)scale, scores, out + row * D);
        free(scores);
        free(qd);
    }
    return err;
}

int oracle_paged_prefill_bf16(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              const int32_t *q_offsets, int S, int Hq, int Hkv, int D, int BS,
                              int MB, int64_t NB, float scale, double *out)
{
    kv_src src = {KV_BF16, k_cache, v_cache, NULL, NULL};
    return prefill_common(q, &src, block_tables, context_lens, q_offsets, S, Hq, Hkv, D, BS, MB,
                          NB, scale, out);
}

/* The same chunked prefill over an int8 cache (element = code * its (slot, kv
 * head) scale, ybb.press page section 6.1) or an FP8 E4M3 cache (element = the
 * code's value). */
int oracle_paged_prefill_int8(const uint16_t *q, const int8_t *k_cache, const int8_t *v_cache,
                              const float *k_scales, const float *v_scales,
                              const int32_t *block_tables, const int32_t *context_lens,
                              const int32_t *q_offsets, int S, int Hq, int Hkv, int D, int BS,
                              int MB, int64_t NB, float scale, double *out)
{
    kv_src src = {KV_INT8, k_cache, v_cache, k_scales, v_scales};
    return prefill_common(q, &src, block_tables, context_lens, q_offsets, S, Hq, Hkv, D, BS, MB,
                          NB, scale, out);
}

int oracle_paged_prefill_fp8(const uint16_t *q, const uint8_t *k_cache, const uint8_t *v_cache,
                             const int32_t *block_tables, const int32_t *context_lens,
                             const int32_t *q_offsets, int S, int Hq, int Hkv, int D, int BS,
                             int MB, int64_t NB, float scale, double *out)
{
    kv_src src = {KV_FP8, k_cache, v_cache, NULL, NULL};
    return prefill_common(q, &src, block_tables, context_lens, q_offsets, S, Hq, Hkv, D, BS, MB,
                          NB, scale, out);
}

/*
 * PagedEviction, prefill phase (blog.hotdry.top page, section "PagedEviction
 * 块级驱逐机制": in the prefill phase each token's importance is computed and
 * the low-scoring tokens are evicted down to the budget; compression there is
 * per token, not per block).
 *
 * Reading taken: for each sequence with n = context_lens[s] > budget, the
 * tokens are ranked by importance, highest first (a NaN importance ranks
 * above every number, as the decode-phase rule never evicts a NaN block; equal
 * importances, -0 and +0 included, rank by position, earlier first); the
 * first `budget` of that ranking are kept, in their original order, and moved
 * to logical positions 0 .. budget-1 of the same sequence.  A kept token takes
 * its whole cache row with it: its K and V rows (all kv heads; any element
 * type, moved as bytes), its int8 scales when present, and its importance.
 * context_lens[s] becomes budget.  Slots at logical positions >= budget, and
 * every other sequence, are left as they were; the block table is not
 * changed (entries from ceil(budget / BS) on no longer belong to the context).
 *
 * Plain form: the ranking is a full sort of (importance, position) pairs,
 * and the kept rows are copied out to a buffer before any is written back.
 * Checked caller contract: valid and pairwise distinct block ids for every
 * logical block of every compressed sequence.
 */
typedef struct {
    float score;
    int32_t pos;
} ranked_token;

static int rank_cmp(const void *pa, const void *pb)
{
    const ranked_token *a = (const ranked_token *)pa, *b = (const ranked_token *)pb;
    const int an = isnan(a->score), bn = isnan(b->score);
    if (an != bn) return an ? -1 : 1;                 /* NaN first */
    if (!an && a->score != b->score) return a->score > b->score ? -1 : 1;   /* higher first */
    return (a->pos > b->pos) - (a->pos < b->pos);     /* then earlier first */
}

static int int_cmp(const void *pa, const void *pb)
{
    const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

int oracle_compress_prefill(uint8_t *k_cache, uint8_t *v_cache, int64_t row_bytes, float *k_scales,
                            float *v_scales, int Hkv, float *scores, const int32_t *block_tables,
                            int32_t *context_lens, int S, int MB, int BS, int64_t NB, int budget)
{
    if (!k_cache || !v_cache || !scores || !block_tables || !context_lens) return ORC_ERR_ARG;
    if (S < 0 || MB <= 0 || BS <= 0 || NB < 0 || row_bytes <= 0 || budget < 0) return ORC_ERR_ARG;
    if ((k_scales == NULL) != (v_scales == NULL) || (k_scales && Hkv <= 0)) return ORC_ERR_ARG;
    unsigned char *used = (unsigned char *)calloc((size_t)(NB > 0 ? NB : 1), 1);
    if (!used) return ORC_ERR_NOMEM;
    int rc = ORC_OK;
    for (int s = 0; s < S && rc == ORC_OK; ++s) {
        const int n = context_lens[s];
        if (n < 0 || (int64_t)n > (int64_t)MB * BS) rc = ORC_ERR_TABLE;
        else if (n > budget)
            for (int j = 0; j < (n + BS - 1) / BS; ++j) {
                const int32_t b = block_tables[(int64_t)s * MB + j];
                if (b < 0 || (int64_t)b >= NB || used[b]) { rc = ORC_ERR_TABLE; break; }
                used[b] = 1;
            }
    }
    free(used);
    if (rc != ORC_OK) return rc;
    const int ns = k_scales ? Hkv : 0;
    for (int s = 0; s < S; ++s) {
        const int n = context_lens[s];
        if (n <= budget) continue;
        const int32_t *row = block_tables + (int64_t)s * MB;
        ranked_token *rk = (ranked_token *)malloc((size_t)n * sizeof *rk);
        int32_t *keep = (int32_t *)malloc((size_t)(budget > 0 ? budget : 1) * sizeof *keep);
        uint8_t *kb = (uint8_t *)malloc((size_t)(budget > 0 ? budget : 1) * (size_t)row_bytes);
        uint8_t *vb = (uint8_t *)malloc((size_t)(budget > 0 ? budget : 1) * (size_t)row_bytes);
        float *fb = (float *)malloc((size_t)(budget > 0 ? budget : 1) * (size_t)(2 * ns + 1) * sizeof(float));
        if (!rk || !keep || !kb || !vb || !fb) {
            free(rk); free(keep); free(kb); free(vb); free(fb);
            return ORC_ERR_NOMEM;
        }
        for (int t = 0; t < n; ++t) {
            const int64_t slot = (int64_t)row[t / BS] * BS + t % BS;
            rk[t].score = scores[slot];
            rk[t].pos = t;
        }
        qsort(rk, (size_t)n, sizeof *rk, rank_cmp);
        for (int j = 0; j < budget; ++j) keep[j] = rk[j].pos;
        qsort(keep, (size_t)budget, sizeof *keep, int_cmp);
        /* copy the kept rows out, then write them to positions 0 .. budget-1 */
        for (int j = 0; j < budget; ++j) {
            const int t = keep[j];
            const int64_t slot = (int64_t)row[t / BS] * BS + t % BS;
            memcpy(kb + (size_t)j * row_bytes, k_cache + slot * row_bytes, (size_t)row_bytes);
            memcpy(vb + (size_t)j * row_bytes, v_cache + slot * row_bytes, (size_t)row_bytes);
            float *f = fb + (size_t)j * (2 * ns + 1);
            for (int g = 0; g < ns; ++g) {
                f[g] = k_scales[slot * Hkv + g];
                f[ns + g] = v_scales[slot * Hkv + g];
            }
            f[2 * ns] = scores[slot];
        }
        for (int j = 0; j < budget; ++j) {
            const int64_t slot = (int64_t)row[j / BS] * BS + j % BS;
            memcpy(k_cache + slot * row_bytes, kb + (size_t)j * row_bytes, (size_t)row_bytes);
            memcpy(v_cache + slot * row_bytes, vb + (size_t)j * row_bytes, (size_t)row_bytes);
            const float *f = fb + (size_t)j * (2 * ns + 1);
            for (int g = 0; g < ns; ++g) {
                k_scales[slot * Hkv + g] = f[g];
                v_scales[slot * Hkv + g] = f[ns + g];
            }
            scores[slot] = f[2 * ns];
        }
        context_lens[s] = budget;
        free(rk); free(keep); free(kb); free(vb); free(fb);
    }
    return ORC_OK;
}
