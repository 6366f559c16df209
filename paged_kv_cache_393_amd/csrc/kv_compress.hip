// kv_compress.hip -- PagedEviction's prefill phase on gfx950 (CDNA4) behind
// the C-ABI of include/paged_kv_evict.h: token-level compression of each
// sequence's paged cache down to a budget (page "KV缓存内存布局优化：分页策略、
// 量化压缩与动态驱逐的工程实践", section "PagedEviction 块级驱逐机制": in the
// prefill phase every token's importance is computed and the low-scoring
// tokens are evicted until the budget is met).
//
// Ranking (the reading documented with the entry points): importance highest
// first, a NaN above every number, equal importances (-0 and +0 included) by
// position, earlier first.  The kept tokens keep their order and move to
// logical positions 0 .. budget-1 of their own sequence, in place.
//
// Two kernels:
//   * select: one workgroup per sequence.  Each importance maps to a 32-bit
//     key whose unsigned order is the ranking (without the position); a
//     4-pass MSB-first radix select over 8-bit digits finds the key T of the
//     budget-th token and how many tokens of key T are kept (LDS histogram;
//     on the first digit, which a sequence's keys mostly share, the lanes of
//     a wave with equal digits add to its bin once); a last pass in
//     position order marks the kept tokens (key > T, or key == T among the
//     first ones) and writes their positions, compacted, to the workspace.
//     Keys sit in LDS when the context fits, else in the workspace, written
//     once and read back by every pass.
//   * move: one workgroup per (kv head, sequence) -- or per slice of a head's
//     row -- moves that part of each kept row (K, V, int8 scales; the
//     importance with head 0).  Kept
//     token j comes from position t_j >= j, so a row is only ever overwritten
//     by a token at a lower position: destinations are taken in chunks, all
//     reads of a chunk complete (vmcnt(0), barrier) before its writes, and a
//     chunk's destinations lie below every later chunk's sources.  Tokens
//     already in place (t_j == j, the common prefix) are not touched.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_kv_evict.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kLdsKeys = 12288;      // contexts up to this many tokens keep their keys in LDS
constexpr int kMoveThreads = 256;
#ifndef KC_ROUNDS
#define KC_ROUNDS 8
#endif
#ifndef KC_SLICE
#define KC_SLICE 256
#endif
constexpr int kMoveRounds = KC_ROUNDS;   // 16-B pieces in flight per thread and chunk
constexpr int kSliceBytes = KC_SLICE;    // bytes of a head row one workgroup moves (whole lines)
constexpr int kMoveWindow = 1024;        // kept tokens whose slots are resolved at once

struct CompressParams {
    void *k;
    void *v;
    float *k_scales;        // int8 only (else null)
    float *v_scales;
    float *scores;          // [NB, bs]
    const int32_t *block_tables;
    int32_t *context_lens;
    int32_t *keep;          // workspace: [S, budget] kept positions
    int32_t *ctx;           // workspace: [S] context length at the call
    uint32_t *keys;         // workspace: [S, max_ctx] ranking keys of contexts too long for LDS
    int hkv;
    int head_bytes;         // bytes of one kv head's row: head_dim * element size
    int slices;             // workgroups per head row: head_bytes / slice bytes
    int block_size;
    int max_blocks_per_seq;
    int max_ctx;
    int budget;
};

// Ranking key of an importance: larger key = ranked higher (position aside).
__device__ __forceinline__ uint32_t rank_key(float x) {
    if (x != x) return 0xFFFFFFFFu;                  // NaN above everything
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;                    // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int64_t slot_of(const int32_t *row, int t, int bs) {
    return (int64_t)row[t / bs] * bs + t % bs;
}

__global__ __launch_bounds__(kSelThreads) void compress_select_kernel(CompressParams p) {
    __shared__ uint32_t lds_key[kLdsKeys];
    __shared__ uint32_t hist[256];
    __shared__ int lds_pick[2];
    __shared__ int lds_wave[2][kSelWaves];
    const int s = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = min(max(p.context_lens[s], 0), p.max_ctx);
    if (tid == 0) p.ctx[s] = n;
    const int budget = p.budget;
    if (n <= budget || budget == 0) return;
    const int bs = p.block_size;
    const int32_t *row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const bool in_lds = n <= kLdsKeys;
    // Keys of a context too long for LDS go to this sequence's workspace row.
    uint32_t *gkeys = p.keys + (int64_t)s * p.max_ctx;
    {
        // four tokens per thread at a time: their table and score loads in flight together
        for (int c0 = 0; c0 < n; c0 += 4 * kSelThreads) {
            int64_t slot[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = c0 + u * kSelThreads + tid;
                slot[u] = t < n ? slot_of(row, t, bs) : 0;
            }
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = c0 + u * kSelThreads + tid;
                x[u] = t < n ? p.scores[slot[u]] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = c0 + u * kSelThreads + tid;
                if (t < n) {
                    if (in_lds) lds_key[t] = rank_key(x[u]);
                    else gkeys[t] = rank_key(x[u]);
                }
            }
        }
        // the workgroup's global key stores are complete and visible to all its waves
        if (!in_lds) __threadfence_block();
    }
    auto key_at = [&](int t) __attribute__((always_inline)) {
        return in_lds ? lds_key[t] : gkeys[t];
    };

    // Radix select of the budget-th largest key, 8 bits a pass from the top.
    uint32_t prefix = 0, mask = 0;
    int need = budget;   // keys still to take among those matching the prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        if (shift == 24) {
            // first digit: the keys of a sequence mostly share it, so lanes of
            // a wave with the same digit add to its bin once
            for (int c0 = 0; c0 < n; c0 += kSelThreads) {
                const int t = c0 + tid;
                const uint32_t d = t < n ? key_at(t) >> 24 : 0u;
                uint64_t todo = __ballot(t < n);
                while (todo) {
                    const uint32_t dl = __shfl(d, __builtin_ctzll(todo));
                    const uint64_t same = __ballot(t < n && d == dl);
                    if (lane == __builtin_ctzll(todo)) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
                    todo &= ~same;
                }
            }
        } else {
            for (int c0 = 0; c0 < n; c0 += 4 * kSelThreads) {
                uint32_t k[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = c0 + u * kSelThreads + tid;
                    k[u] = t < n ? key_at(t) : 0u;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = c0 + u * kSelThreads + tid;
                    if (t < n && (k[u] & mask) == prefix) atomicAdd(&hist[(k[u] >> shift) & 255u], 1u);
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane L holds bins 4L .. 4L+3; count the keys above each bin
            uint32_t c[4];
            for (int b = 0; b < 4; ++b) c[b] = hist[4 * lane + b];
            const uint32_t mine = c[0] + c[1] + c[2] + c[3];
            // keys in the bins of higher lanes (every lane takes part in each shuffle)
            uint32_t incl = mine;   // inclusive suffix sum over lanes lane .. 63
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_down(incl, off);
                if (lane + off < 64) incl += o;
            }
            uint32_t above = incl - mine;
            for (int b = 3; b >= 0; --b) {
                if (above < (uint32_t)need && (uint32_t)need <= above + c[b]) {
                    lds_pick[0] = 4 * lane + b;
                    lds_pick[1] = (int)above;
                }
                above += c[b];
            }
        }
        __syncthreads();
        const int digit = lds_pick[0];
        need -= lds_pick[1];
        prefix |= (uint32_t)digit << shift;
        mask |= 0xFFu << shift;
        __syncthreads();   // lds_pick and hist are rewritten by the next pass
    }
    const uint32_t T = prefix;   // key of the budget-th token; `need` tokens of key T are kept

    // Mark and compact in position order.
    int eq_before = 0, kept_before = 0;
    int32_t *keep = p.keep + (int64_t)s * budget;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t k_next = tid < n ? key_at(tid) : 0u;
    for (int c0 = 0; c0 < n; c0 += kSelThreads) {
        const int t = c0 + tid;
        const uint32_t k = k_next;   // this chunk's key; the next one's load is in flight meanwhile
        k_next = t + kSelThreads < n ? key_at(t + kSelThreads) : 0u;
        const bool eq = t < n && k == T;
        const uint64_t eq_bal = __ballot(eq);
        if (lane == 0) lds_wave[0][wave] = __popcll(eq_bal);
        __syncthreads();
        int eq_rank = eq_before + __popcll(eq_bal & lt_mask), eq_total = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            const int cnt = lds_wave[0][w];
            if (w < wave) eq_rank += cnt;
            eq_total += cnt;
        }
        const bool kept = t < n && (k > T || (eq && eq_rank < need));
        const uint64_t kp_bal = __ballot(kept);
        if (lane == 0) lds_wave[1][wave] = __popcll(kp_bal);
        __syncthreads();
        int pos = kept_before + __popcll(kp_bal & lt_mask), kp_total = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            const int cnt = lds_wave[1][w];
            if (w < wave) pos += cnt;
            kp_total += cnt;
        }
        if (kept && pos < budget) keep[pos] = t;
        eq_before += eq_total;
        kept_before += kp_total;
        __syncthreads();   // lds_wave is rewritten by the next chunk
    }
}

// Moves slice blockIdx.x % slices of kv head blockIdx.x / slices of the kept
// rows of sequence blockIdx.y.  The source and destination slots of a window
// of kept tokens are resolved once into LDS (their keep-list and table loads
// in flight together), so a chunk waits only for its own K/V loads.
template <bool kScales>
__global__ __launch_bounds__(kMoveThreads) void compress_move_kernel(CompressParams p) {
    __shared__ int64_t lds_src[kMoveWindow];   // source slot of kept token w0 + i, or -1 (in place)
    __shared__ int64_t lds_dst[kMoveWindow];
    const int g = blockIdx.x / p.slices;
    const int slice = blockIdx.x - g * p.slices;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int n = p.ctx[s];
    const int budget = p.budget;
    if (n <= budget) return;
    const int bs = p.block_size;
    const int32_t *row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const int32_t *keep = p.keep + (int64_t)s * budget;
    const int pieces = p.head_bytes / p.slices / 16;   // 16-B pieces of this slice
    const int tok_per_round = kMoveThreads / pieces;
    const int piece = tid % pieces;
    const int64_t row_bytes = (int64_t)p.hkv * p.head_bytes;
    const int64_t col = (int64_t)g * p.head_bytes + (int64_t)slice * pieces * 16 + piece * 16;
    char *kbase = (char *)p.k + col;
    char *vbase = (char *)p.v + col;
    const bool lead = slice == 0 && piece == 0;     // moves the per-token floats
    for (int w0 = 0; w0 < budget; w0 += kMoveWindow) {
        const int wn = min(kMoveWindow, budget - w0);
        __syncthreads();   // the previous window's slots have been read
        constexpr int kPer = kMoveWindow / kMoveThreads;
        int tk[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = u * kMoveThreads + tid;
            tk[u] = i < wn ? keep[w0 + i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = u * kMoveThreads + tid;
            const int j = w0 + i;
            const bool mv = i < wn && tk[u] > j && tk[u] < n;   // kept token tk moves down to j
            if (i < wn) {
                lds_src[i] = mv ? slot_of(row, tk[u], bs) : -1;
                lds_dst[i] = mv ? slot_of(row, j, bs) : -1;
            }
        }
        __syncthreads();
        for (int c0 = 0; c0 < wn; c0 += kMoveRounds * tok_per_round) {
            u32x4_t kr[kMoveRounds], vr[kMoveRounds];
            float ks[kMoveRounds], vs[kMoveRounds], sc[kMoveRounds];
            int64_t src[kMoveRounds], dst[kMoveRounds];
#pragma unroll
            for (int r = 0; r < kMoveRounds; ++r) {
                const int i = c0 + r * tok_per_round + tid / pieces;
                src[r] = i < wn ? lds_src[i] : -1;
                dst[r] = i < wn ? lds_dst[i] : -1;
            }
#pragma unroll
            for (int r = 0; r < kMoveRounds; ++r) {
                if (src[r] < 0) continue;
                const int64_t off = src[r] * row_bytes;
                kr[r] = __builtin_nontemporal_load((const u32x4_t *)(kbase + off));
                vr[r] = __builtin_nontemporal_load((const u32x4_t *)(vbase + off));
                if (lead) {
                    if constexpr (kScales) {
                        ks[r] = p.k_scales[src[r] * p.hkv + g];
                        vs[r] = p.v_scales[src[r] * p.hkv + g];
                    }
                    if (g == 0) sc[r] = p.scores[src[r]];
                }
            }
            // Every read of this chunk has returned before any thread writes.
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
#pragma unroll
            for (int r = 0; r < kMoveRounds; ++r) {
                if (src[r] < 0) continue;
                const int64_t off = dst[r] * row_bytes;
                *(u32x4_t *)(kbase + off) = kr[r];
                *(u32x4_t *)(vbase + off) = vr[r];
                if (lead) {
                    if constexpr (kScales) {
                        p.k_scales[dst[r] * p.hkv + g] = ks[r];
                        p.v_scales[dst[r] * p.hkv + g] = vs[r];
                    }
                    if (g == 0) p.scores[dst[r]] = sc[r];
                }
            }
        }
    }
    if (blockIdx.x == 0 && tid == 0) p.context_lens[s] = budget;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

size_t keep_bytes(int64_t S, int64_t budget) { return (size_t)(((S * budget * 4) + 255) & ~(int64_t)255); }
size_t ctx_bytes(int64_t S) { return (size_t)(((S * 4) + 255) & ~(int64_t)255); }
// Key rows are needed only for contexts longer than the LDS holds.
size_t key_bytes(int64_t S, int64_t max_ctx) {
    return max_ctx > kLdsKeys ? (size_t)(((S * max_ctx * 4) + 255) & ~(int64_t)255) : 0;
}

int compress_common(bool int8, int elem, void *k, void *v, float *ks, float *vs, float *scores,
                    const int32_t *bt, int32_t *cl, int32_t budget, const pa_score_shape *sh,
                    void *ws, size_t ws_bytes, void *stream) {
    if (!sh) return PA_ERR_NULL;
    if (sh->num_seqs < 0 || sh->num_kv_heads < 1 || sh->block_size < 1 ||
        sh->max_blocks_per_seq < 1 || sh->num_blocks < 1 || budget < 0)
        return PA_ERR_SHAPE;
    if (sh->head_dim != 64 && sh->head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (sh->block_size > 4096 || sh->num_seqs > 65535 || sh->num_kv_heads > 32767) return PA_ERR_UNSUPPORTED;
    const int64_t max_ctx = (int64_t)sh->max_blocks_per_seq * sh->block_size;
    if (max_ctx >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    if (sh->num_seqs == 0) return PA_OK;
    if (!k || !v || !scores || !bt || !cl) return PA_ERR_NULL;
    if (int8 && (!ks || !vs)) return PA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v)) return PA_ERR_ALIGNMENT;
    const size_t need = paged_kv_compress_workspace_bytes(sh, budget);
    if (!ws || ws_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned16(ws)) return PA_ERR_ALIGNMENT;
    CompressParams p;
    p.k = k;
    p.v = v;
    p.k_scales = int8 ? ks : nullptr;
    p.v_scales = int8 ? vs : nullptr;
    p.scores = scores;
    p.block_tables = bt;
    p.context_lens = cl;
    p.keep = (int32_t *)ws;
    p.ctx = (int32_t *)((char *)ws + keep_bytes(sh->num_seqs, budget));
    p.keys = (uint32_t *)((char *)ws + keep_bytes(sh->num_seqs, budget) + ctx_bytes(sh->num_seqs));
    p.hkv = sh->num_kv_heads;
    p.head_bytes = sh->head_dim * elem;
    p.slices = p.head_bytes > kSliceBytes ? p.head_bytes / kSliceBytes : 1;
    p.block_size = sh->block_size;
    p.max_blocks_per_seq = sh->max_blocks_per_seq;
    p.max_ctx = (int)max_ctx;
    p.budget = budget;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(compress_select_kernel, dim3((unsigned)sh->num_seqs), dim3(kSelThreads), 0, st, p);
    const dim3 mgrid((unsigned)(sh->num_kv_heads * p.slices), (unsigned)sh->num_seqs);
    if (int8) hipLaunchKernelGGL(compress_move_kernel<true>, mgrid, dim3(kMoveThreads), 0, st, p);
    else hipLaunchKernelGGL(compress_move_kernel<false>, mgrid, dim3(kMoveThreads), 0, st, p);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t paged_kv_compress_workspace_bytes(const pa_score_shape *shape, int32_t budget) {
    if (!shape || shape->num_seqs < 0 || budget < 0) return 0;
    return keep_bytes(shape->num_seqs, budget) + ctx_bytes(shape->num_seqs) +
           key_bytes(shape->num_seqs, (int64_t)shape->max_blocks_per_seq * shape->block_size);
}

int paged_kv_compress_prefill(void *k_cache, void *v_cache, float *scores,
                              const int32_t *block_tables, int32_t *context_lens, int32_t budget,
                              const pa_score_shape *shape, void *workspace, size_t workspace_bytes,
                              void *stream) {
    return compress_common(false, 2, k_cache, v_cache, nullptr, nullptr, scores, block_tables,
                           context_lens, budget, shape, workspace, workspace_bytes, stream);
}

int paged_kv_compress_prefill_int8(int8_t *k_cache, int8_t *v_cache, float *k_scales,
                                   float *v_scales, float *scores, const int32_t *block_tables,
                                   int32_t *context_lens, int32_t budget,
                                   const pa_score_shape *shape, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    return compress_common(true, 1, k_cache, v_cache, k_scales, v_scales, scores, block_tables,
                           context_lens, budget, shape, workspace, workspace_bytes, stream);
}

int paged_kv_compress_prefill_fp8(uint8_t *k_cache, uint8_t *v_cache, float *scores,
                                  const int32_t *block_tables, int32_t *context_lens,
                                  int32_t budget, const pa_score_shape *shape, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return compress_common(false, 1, k_cache, v_cache, nullptr, nullptr, scores, block_tables,
                           context_lens, budget, shape, workspace, workspace_bytes, stream);
}

}  // extern "C"
