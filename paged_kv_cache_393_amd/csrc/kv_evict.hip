// kv_evict.hip -- PagedEviction on gfx950 (CDNA4) behind the C-ABI of
// include/paged_kv_evict.h: token importance ||V|| / ||K|| over the paged
// cache, and the decode-phase eviction of the full block of lowest mean
// importance (page "KV缓存内存布局优化：分页策略、量化压缩与动态驱逐的工程实践",
// section "PagedEviction 块级驱逐机制").
//
// Scoring is a streaming reduction over the same bytes decode reads, so it is
// shaped for HBM: one workgroup per (sequence, logical block); a group of 16
// lanes (8 when a token row has only 64 elements) owns one token and walks its
// row -- all kv heads side by side, adjacent in memory -- in 8-element chunks,
// summing the squares of K and V; the group's two sums meet through DPP lane
// moves and one lane writes the score at the token's slot.  int8 squares are
// exact integer dot products (v_dot4) scaled by the head's squared scale; fp8
// codes are converted exactly with v_cvt_pk_f32_fp8.
//
// Eviction is latency work on a few KB per sequence: one workgroup per
// sequence forms each full block's mean in double, adding its scores in slot
// order (so the decision is bit-identical to a sequential reference given the
// same fp32 scores), reduces (mean, block) to the first minimum, and shifts
// the table row down over the victim.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_kv_evict.h"

namespace {

constexpr int kThreads = 256;
enum ScoreKind : int { kScoreBf16 = 0, kScoreInt8 = 1, kScoreFp8 = 2 };

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Cache rows are read once per call: non-temporal loads (nt), so the
// streamed lines are not kept in the caches.
template <typename T>
__device__ __forceinline__ T stream_load(const char *p) {
    return __builtin_nontemporal_load((const T *)p);
}

struct ScoreParams {
    const void *k;
    const void *v;
    const float *k_scales;   // int8 only
    const float *v_scales;
    const int32_t *block_tables;
    const int32_t *token_begin;   // may be null
    const int32_t *context_lens;
    float *scores;               // [NB, bs]
    int hkv;
    int head_dim;
    int chunks;                  // 8-element chunks per token row: hkv * head_dim / 8
    int block_size;
    int max_blocks_per_seq;
};

// A DPP lane move inside each 16-lane row (kCtrl: a gfx9 dpp_ctrl value).
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of L lanes (8 or 16), left in every lane of the
// group: quad permutations xor 1 and xor 2, then the half-row mirror (lane
// i <-> 7 - i) and the row mirror (lane i <-> 15 - i), each of which pairs the
// two halves of the span summed so far.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(L == 8 || L == 16, "groups of 8 or 16 lanes");
    v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v);   // row_half_mirror
    if constexpr (L == 16) v += dpp_move<0x140>(v);   // row_mirror
    return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float sumsq_bf16x2(uint32_t w, float acc) {
    const float a = bf16_lo(w), b = bf16_hi(w);
    return fmaf(b, b, fmaf(a, a, acc));
}

__device__ __forceinline__ float sumsq_fp8x4(uint32_t w, float acc) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    acc = fmaf(lo.x, lo.x, acc);
    acc = fmaf(lo.y, lo.y, acc);
    acc = fmaf(hi.x, hi.x, acc);
    return fmaf(hi.y, hi.y, acc);
}

template <int KIND, int L>
__global__ __launch_bounds__(kThreads) void token_scores_kernel(ScoreParams p) {
    constexpr int kTokensPerPass = kThreads / L;
    const int j = blockIdx.x;     // logical block
    const int s = blockIdx.y;     // sequence
    const int bs = p.block_size;
    const int n = p.context_lens[s];
    const int t_lo = max(j * bs, p.token_begin ? p.token_begin[s] : 0);
    const int t_hi = min(n, (j + 1) * bs);
    if (t_lo >= t_hi) return;
    const int64_t phys = p.block_tables[(int64_t)s * p.max_blocks_per_seq + j];
    const int li = threadIdx.x % L;
    constexpr int kElem = KIND == kScoreBf16 ? 2 : 1;
    const int64_t row_elems = (int64_t)p.chunks * 8;

    // Every lane of a token's group has the same t, so the group takes each
    // branch together and the lane moves only read lanes that are active.
    for (int t = j * bs + (int)(threadIdx.x / L); t < t_hi; t += kTokensPerPass) {
        if (t < t_lo) continue;
        const int r = t - j * bs;
        const int64_t slot = phys * bs + r;
        const char *krow = (const char *)p.k + slot * row_elems * kElem;
        const char *vrow = (const char *)p.v + slot * row_elems * kElem;
        float kk = 0.f, vv = 0.f;
        for (int c = li; c < p.chunks; c += L) {
            if constexpr (KIND == kScoreBf16) {
                const u32x4_t kw = stream_load<u32x4_t>(krow + c * 16);
                const u32x4_t vw = stream_load<u32x4_t>(vrow + c * 16);
                kk = sumsq_bf16x2(kw.w, sumsq_bf16x2(kw.z, sumsq_bf16x2(kw.y, sumsq_bf16x2(kw.x, kk))));
                vv = sumsq_bf16x2(vw.w, sumsq_bf16x2(vw.z, sumsq_bf16x2(vw.y, sumsq_bf16x2(vw.x, vv))));
            } else if constexpr (KIND == kScoreFp8) {
                const u32x2_t kw = stream_load<u32x2_t>(krow + c * 8);
                const u32x2_t vw = stream_load<u32x2_t>(vrow + c * 8);
                kk = sumsq_fp8x4(kw.y, sumsq_fp8x4(kw.x, kk));
                vv = sumsq_fp8x4(vw.y, sumsq_fp8x4(vw.x, vv));
            } else {
                const u32x2_t kw = stream_load<u32x2_t>(krow + c * 8);
                const u32x2_t vw = stream_load<u32x2_t>(vrow + c * 8);
                // sum of the 8 codes' squares: exact (at most 8 * 128^2)
                const int ksq = __builtin_amdgcn_sdot4((int)kw.y, (int)kw.y,
                                                       __builtin_amdgcn_sdot4((int)kw.x, (int)kw.x, 0, false), false);
                const int vsq = __builtin_amdgcn_sdot4((int)vw.y, (int)vw.y,
                                                       __builtin_amdgcn_sdot4((int)vw.x, (int)vw.x, 0, false), false);
                const int g = (c * 8) / p.head_dim;   // the chunk lies in one head
                const float ks = p.k_scales[slot * p.hkv + g];
                const float vs = p.v_scales[slot * p.hkv + g];
                kk = fmaf((float)ksq, ks * ks, kk);
                vv = fmaf((float)vsq, vs * vs, vv);
            }
        }
        kk = group_sum<L>(kk);
        vv = group_sum<L>(vv);
        if (li == 0) p.scores[slot] = __builtin_sqrtf(vv) / __builtin_sqrtf(kk);
    }
}

struct EvictParams {
    const float *scores;
    int32_t *block_tables;
    int32_t *context_lens;
    const int32_t *evict_mask;
    int32_t *evicted;
    int block_size;
    int max_blocks_per_seq;
};

// (mean, block) candidates: a beats b when b is empty, or a's mean is smaller,
// or the means are equal and a's block comes first.  NaN means never enter.
__device__ __forceinline__ bool beats(double am, int aj, double bm, int bj) {
    if (aj < 0) return false;
    if (bj < 0) return true;
    return am < bm || (am == bm && aj < bj);
}

__global__ __launch_bounds__(kThreads) void evict_lowest_block_kernel(EvictParams p) {
    __shared__ double lds_m[kThreads / 64];
    __shared__ int lds_j[kThreads / 64];
    __shared__ int lds_victim;
    const int s = blockIdx.x;
    const int bs = p.block_size;
    const int n = p.context_lens[s];
    const int n_full = n / bs;
    if (!p.evict_mask[s] || n_full <= 0) {
        if (threadIdx.x == 0) p.evicted[s] = -1;
        return;
    }
    int32_t *row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;

    double best_m = 0.0;
    int best_j = -1;
    for (int j = threadIdx.x; j < n_full; j += kThreads) {
        const float *blk = p.scores + (int64_t)row[j] * bs;
        double sum = 0.0;
        for (int r = 0; r < bs; ++r) sum += (double)blk[r];
        const double mean = sum / bs;
        if (mean != mean) continue;                    // NaN
        if (beats(mean, j, best_m, best_j)) {
            best_m = mean;
            best_j = j;
        }
    }
    for (int off = 1; off < 64; off <<= 1) {
        const double om = __shfl_xor(best_m, off);
        const int oj = __shfl_xor(best_j, off);
        if (beats(om, oj, best_m, best_j)) {
            best_m = om;
            best_j = oj;
        }
    }
    const int wave = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) {
        lds_m[wave] = best_m;
        lds_j[wave] = best_j;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double m = lds_m[0];
        int jv = lds_j[0];
        for (int w = 1; w < kThreads / 64; ++w)
            if (beats(lds_m[w], lds_j[w], m, jv)) {
                m = lds_m[w];
                jv = lds_j[w];
            }
        lds_victim = jv < 0 ? 0 : jv;
    }
    __syncthreads();
    const int victim = lds_victim;
    const int nblk = (n + bs - 1) / bs;
    const int32_t victim_id = row[victim];
    __syncthreads();   // every thread has read the victim's id before the row moves
    // Shift entries victim+1 .. nblk-1 down by one, kThreads at a time: all
    // reads of a round finish (barrier) before its writes.
    for (int base = victim; base < nblk - 1; base += kThreads) {
        const int j = base + threadIdx.x;
        const int32_t next = j < nblk - 1 ? row[j + 1] : 0;
        __syncthreads();
        if (j < nblk - 1) row[j] = next;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        row[nblk - 1] = -1;
        p.context_lens[s] = n - bs;
        p.evicted[s] = victim_id;
    }
}

bool aligned(const void *ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

int check_shape(const pa_score_shape *sh) {
    if (!sh) return PA_ERR_NULL;
    if (sh->num_seqs < 0 || sh->num_kv_heads < 1 || sh->block_size < 1 ||
        sh->max_blocks_per_seq < 1 || sh->num_blocks < 1)
        return PA_ERR_SHAPE;
    if (sh->head_dim != 64 && sh->head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (sh->block_size > 4096 || sh->num_seqs > 65535) return PA_ERR_UNSUPPORTED;
    if ((int64_t)sh->max_blocks_per_seq * sh->block_size >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

int scores_common(int kind, const void *k, const void *v, const float *ks, const float *vs,
                  const int32_t *bt, const int32_t *tb, const int32_t *cl, float *scores,
                  const pa_score_shape *sh, void *stream) {
    int rc = check_shape(sh);
    if (rc != PA_OK) return rc;
    if (sh->num_seqs == 0) return PA_OK;
    if (!k || !v || !bt || !cl || !scores) return PA_ERR_NULL;
    if (kind == kScoreInt8 && (!ks || !vs)) return PA_ERR_NULL;
    if (!aligned(k, kind == kScoreBf16 ? 16 : 8) || !aligned(v, kind == kScoreBf16 ? 16 : 8) ||
        !aligned(scores, 4))
        return PA_ERR_ALIGNMENT;
    ScoreParams p;
    p.k = k;
    p.v = v;
    p.k_scales = ks;
    p.v_scales = vs;
    p.block_tables = bt;
    p.token_begin = tb;
    p.context_lens = cl;
    p.scores = scores;
    p.hkv = sh->num_kv_heads;
    p.head_dim = sh->head_dim;
    p.chunks = sh->num_kv_heads * sh->head_dim / 8;
    p.block_size = sh->block_size;
    p.max_blocks_per_seq = sh->max_blocks_per_seq;
    const dim3 grid((unsigned)sh->max_blocks_per_seq, (unsigned)sh->num_seqs), block(kThreads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool wide = p.chunks >= 16;   // 16 lanes per token, else 8
    switch (kind * 2 + (wide ? 1 : 0)) {
        case 0: hipLaunchKernelGGL((token_scores_kernel<kScoreBf16, 8>), grid, block, 0, st, p); break;
        case 1: hipLaunchKernelGGL((token_scores_kernel<kScoreBf16, 16>), grid, block, 0, st, p); break;
        case 2: hipLaunchKernelGGL((token_scores_kernel<kScoreInt8, 8>), grid, block, 0, st, p); break;
        case 3: hipLaunchKernelGGL((token_scores_kernel<kScoreInt8, 16>), grid, block, 0, st, p); break;
        case 4: hipLaunchKernelGGL((token_scores_kernel<kScoreFp8, 8>), grid, block, 0, st, p); break;
        default: hipLaunchKernelGGL((token_scores_kernel<kScoreFp8, 16>), grid, block, 0, st, p); break;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int paged_kv_token_scores(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                          const int32_t *token_begin, const int32_t *context_lens, float *scores,
                          const pa_score_shape *shape, void *stream) {
    return scores_common(kScoreBf16, k_cache, v_cache, nullptr, nullptr, block_tables, token_begin,
                         context_lens, scores, shape, stream);
}

int paged_kv_token_scores_int8(const int8_t *k_cache, const int8_t *v_cache,
                               const float *k_scales, const float *v_scales,
                               const int32_t *block_tables, const int32_t *token_begin,
                               const int32_t *context_lens, float *scores,
                               const pa_score_shape *shape, void *stream) {
    return scores_common(kScoreInt8, k_cache, v_cache, k_scales, v_scales, block_tables,
                         token_begin, context_lens, scores, shape, stream);
}

int paged_kv_token_scores_fp8(const uint8_t *k_cache, const uint8_t *v_cache,
                              const int32_t *block_tables, const int32_t *token_begin,
                              const int32_t *context_lens, float *scores,
                              const pa_score_shape *shape, void *stream) {
    return scores_common(kScoreFp8, k_cache, v_cache, nullptr, nullptr, block_tables, token_begin,
                         context_lens, scores, shape, stream);
}

int paged_kv_evict_lowest_block(const float *scores, int32_t *block_tables,
                                int32_t *context_lens, const int32_t *evict_mask,
                                int32_t *evicted, const pa_score_shape *shape, void *stream) {
    int rc = check_shape(shape);
    if (rc != PA_OK) return rc;
    if (shape->num_seqs == 0) return PA_OK;
    if (!scores || !block_tables || !context_lens || !evict_mask || !evicted) return PA_ERR_NULL;
    EvictParams p;
    p.scores = scores;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.evict_mask = evict_mask;
    p.evicted = evicted;
    p.block_size = shape->block_size;
    p.max_blocks_per_seq = shape->max_blocks_per_seq;
    hipLaunchKernelGGL(evict_lowest_block_kernel, dim3((unsigned)shape->num_seqs), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), p);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
