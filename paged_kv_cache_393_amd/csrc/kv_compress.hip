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
// Selection, then a move:
//   * select: each importance maps to a 32-bit key whose unsigned order is
//     the ranking (without the position); a 4-pass MSB-first radix select
//     over 8-bit digits finds the key T of the budget-th token and how many
//     tokens of key T are kept; a last pass in position order marks the kept
//     tokens (key > T, or key == T among the first ones) and writes their
//     positions, compacted, to the workspace.  When every context fits in
//     LDS (at most kLdsKeys tokens) one workgroup per sequence does it all
//     (on the first digit, which a sequence's keys mostly share, the lanes of
//     a wave with equal digits add to its bin once).  Longer contexts are
//     split into kChunk-token chunks, one workgroup each, over five launches:
//     keys and first-digit histograms per chunk; one launch per further digit
//     (every chunk picks the previous digit from the summed histograms, then
//     adds its keys' next digits to the sequence's histogram); and the
//     position pass, where a chunk starts from the kept and tied counts of the
//     chunks before it.
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

#include <algorithm>

#include "paged_kv_evict.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kLdsKeys = 12288;      // contexts up to this many tokens: one select workgroup each
constexpr int kChunk = 4096;         // tokens per select workgroup of longer contexts
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
    uint32_t *keys;         // workspace: [S, max_ctx] ranking keys (split select only)
    uint32_t *hist0;        // [S, nch, 256] first-digit histogram of each chunk
    uint32_t *hist12;       // [S, 2, 256] second- and third-digit histograms of each sequence
    int32_t *state;         // [3, S, 2] (key prefix, tokens still to take) after digits 1, 2, 3
    uint32_t *low;          // [S, nch, 257] per chunk: last-digit histogram of the keys that
                            // match the first three digits, then how many keys rank above them
    int nch;                // chunks of the longest context: ceil(max_ctx / kChunk)
    int key_stride;         // keys per sequence row: max_ctx rounded up to a multiple of 4
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

// Wave 0 finds the bin of the need-th largest key from a 256-bin LDS
// histogram of the next digit: lds_pick = (digit, keys in higher bins).  The
// caller synchronises before and after.
__device__ __forceinline__ void pick_digit(const uint32_t *hist, int need, int *lds_pick) {
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
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

// Adds the top digits of this thread's keys (u of them, valid where t < n) to
// an LDS histogram; the lanes of a wave with equal digits add once.
template <int U>
__device__ __forceinline__ void add_top_digits(uint32_t *hist, const uint32_t (&key)[U],
                                               const bool (&ok)[U]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t d = key[u] >> 24;
        uint64_t todo = __ballot(ok[u]);
        while (todo) {
            const uint32_t dl = __shfl(d, __builtin_ctzll(todo));
            const uint64_t same = __ballot(ok[u] && d == dl);
            if (lane == __builtin_ctzll(todo)) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
            todo &= ~same;
        }
    }
}

typedef uint32_t u32x4k_t __attribute__((ext_vector_type(4)));

// Workgroup-wide exclusive prefix sum of one value per thread, and the total,
// through wave shuffles and one LDS slot per wave (lds_w is free on entry and
// must not be rewritten before every thread has returned).
__device__ __forceinline__ int block_excl_scan(int v, int *lds_w, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) lds_w[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int c = lds_w[w];
        if (w < wave) before += c;
        tot += c;
    }
    *total = tot;
    return before + incl - v;
}

// Marks the kept tokens among positions [t0, t1) of one sequence, in
// position order, and writes their positions, compacted, from keep[kept_before]
// on: key > T, or key == T among the first `need` such tokens of the
// sequence (eq_before of them lie before t0).  Each thread takes four
// consecutive positions a round (t0 is a multiple of 4); load4(t) gives the
// keys of positions t .. t+3, and `first` those of the first round.
template <typename Load4>
__device__ __forceinline__ void write_kept(Load4 load4, int t0, int t1, uint32_t T, int need,
                                           int eq_before, int kept_before, int32_t *keep,
                                           int budget, int (*lds_wave)[kSelWaves], u32x4k_t first) {
    const int tid = threadIdx.x;
    u32x4k_t k4 = first;
    for (int base = t0; base < t1; base += 4 * kSelThreads) {
        const int t = base + 4 * tid;
        if (base != t0) k4 = t < t1 ? load4(t) : u32x4k_t{0u, 0u, 0u, 0u};
        const uint32_t k[4] = {k4.x, k4.y, k4.z, k4.w};
        bool eq[4];
        int eqc = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            eq[u] = t + u < t1 && k[u] == T;
            eqc += eq[u] ? 1 : 0;
        }
        int eq_tot;
        int eqr = eq_before + block_excl_scan(eqc, lds_wave[0], &eq_tot);
        bool kept[4];
        int kc = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            kept[u] = t + u < t1 && (k[u] > T || (eq[u] && eqr < need));
            eqr += eq[u] ? 1 : 0;
            kc += kept[u] ? 1 : 0;
        }
        int kp_tot;
        int pos = kept_before + block_excl_scan(kc, lds_wave[1], &kp_tot);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (kept[u]) {
                if (pos < budget) keep[pos] = t + u;
                ++pos;
            }
        }
        eq_before += eq_tot;
        kept_before += kp_tot;
        __syncthreads();   // lds_wave is rewritten by the next round
    }
}

// Select for contexts of at most kLdsKeys tokens: one workgroup per sequence,
// keys in LDS.
__global__ __launch_bounds__(kSelThreads) void compress_select_kernel(CompressParams p) {
    __shared__ __attribute__((aligned(16))) uint32_t lds_key[kLdsKeys];
    __shared__ uint32_t hist[256];
    __shared__ int lds_pick[2];
    __shared__ int lds_wave[2][kSelWaves];
    const int s = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = min(max(p.context_lens[s], 0), p.max_ctx);
    if (tid == 0) p.ctx[s] = n;
    const int budget = p.budget;
    if (n <= budget || budget == 0) return;
    const int bs = p.block_size;
    const int32_t *row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
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
                if (t < n) lds_key[t] = rank_key(x[u]);
            }
        }
    }

    // Radix select of the budget-th largest key, 8 bits a pass from the top.
    uint32_t prefix = 0, mask = 0;
    int need = budget;   // keys still to take among those matching the prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        if (shift == 24) {
            for (int c0 = 0; c0 < n; c0 += kSelThreads) {
                const int t = c0 + tid;
                const uint32_t key[1] = {t < n ? lds_key[t] : 0u};
                const bool ok[1] = {t < n};
                add_top_digits<1>(hist, key, ok);
            }
        } else {
            for (int c0 = 0; c0 < n; c0 += 4 * kSelThreads) {
                uint32_t k[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = c0 + u * kSelThreads + tid;
                    k[u] = t < n ? lds_key[t] : 0u;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = c0 + u * kSelThreads + tid;
                    if (t < n && (k[u] & mask) == prefix) atomicAdd(&hist[(k[u] >> shift) & 255u], 1u);
                }
            }
        }
        __syncthreads();
        pick_digit(hist, need, lds_pick);
        __syncthreads();
        const int digit = lds_pick[0];
        need -= lds_pick[1];
        prefix |= (uint32_t)digit << shift;
        mask |= 0xFFu << shift;
        __syncthreads();   // lds_pick and hist are rewritten by the next pass
    }
    // `prefix` is the key of the budget-th token; `need` tokens of that key are kept.
    // keys past n in the last quad are never compared (t + u < t1)
    auto load4 = [&](int t) __attribute__((always_inline)) {
        return *(const u32x4k_t *)&lds_key[t];
    };
    write_kept(load4, 0, n, prefix, need, 0, 0, p.keep + (int64_t)s * budget, budget, lds_wave,
               4 * tid < n ? load4(4 * tid) : u32x4k_t{0u, 0u, 0u, 0u});
}

// ---- Split select (contexts longer than kLdsKeys): workgroup (c, s) owns
// positions [c * kChunk, min(n, (c + 1) * kChunk)) of sequence s. ----

// Context length and this workgroup's chunk; false when the workgroup has
// nothing to do (no compression, or a chunk past the context end).
__device__ __forceinline__ bool split_chunk(const CompressParams &p, int *n, int *t0, int *t1) {
    const int s = blockIdx.y;
    *n = min(max(p.context_lens[s], 0), p.max_ctx);
    *t0 = blockIdx.x * kChunk;
    *t1 = min(*n, *t0 + kChunk);
    return *n > p.budget && p.budget > 0 && *t0 < *n;
}

// Keys of the chunk (to the workspace) and its first-digit histogram.
__global__ __launch_bounds__(kSelThreads) void compress_split_keys_kernel(CompressParams p) {
    __shared__ uint32_t hist[256];
    const int s = blockIdx.y, tid = threadIdx.x;
    int n, t0, t1;
    const bool work = split_chunk(p, &n, &t0, &t1);
    if (blockIdx.x == 0) {
        if (tid == 0) p.ctx[s] = n;
        // the histograms of digits 2 and 3 are summed by atomics in later launches
        if (tid < 512) p.hist12[(int64_t)s * 512 + tid] = 0u;
    }
    if (!work) return;
    if (tid < 256) hist[tid] = 0u;
    const int32_t *row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    uint32_t *gkeys = p.keys + (int64_t)s * p.key_stride;
    constexpr int U = kChunk / kSelThreads;
    int64_t slot[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kSelThreads + tid;
        ok[u] = t < t1;
        slot[u] = ok[u] ? slot_of(row, t, p.block_size) : 0;
    }
    uint32_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kSelThreads + tid;
        key[u] = ok[u] ? rank_key(p.scores[slot[u]]) : 0u;
        if (ok[u]) gkeys[t] = key[u];
    }
    __syncthreads();
    add_top_digits<U>(hist, key, ok);
    __syncthreads();
    if (tid < 256) p.hist0[((int64_t)s * p.nch + blockIdx.x) * 256 + tid] = hist[tid];
}

// Digit pass `shift` (16 or 8): pick the previous digit from the summed
// histograms, then add the next digit of this chunk's keys that match the
// prefix to the sequence's histogram.  With shift == 0 the chunk keeps its
// own last-digit histogram and the count of keys above the 24-bit prefix.
__global__ __launch_bounds__(kSelThreads) void compress_split_pass_kernel(CompressParams p, int shift) {
    __shared__ uint32_t hist[256];
    __shared__ int lds_pick[2];
    __shared__ uint32_t lds_above;
    const int s = blockIdx.y, tid = threadIdx.x;
    const int S = gridDim.y;
    int n, t0, t1;
    if (!split_chunk(p, &n, &t0, &t1)) return;
    const int pass = shift == 16 ? 0 : (shift == 8 ? 1 : 2);   // digits picked before this pass: pass + 1
    // The chunk's keys do not depend on the digits picked so far: their loads
    // are in flight while the histograms are summed.
    const uint32_t *gkeys = p.keys + (int64_t)s * p.key_stride;
    constexpr int U = kChunk / kSelThreads;
    uint32_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kSelThreads + tid;
        key[u] = t < t1 ? gkeys[t] : 0u;
    }
    // Histogram of the previous digit, summed over the sequence.
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    uint32_t prefix;
    int need;
    if (pass == 0) {
        const int nch = (n + kChunk - 1) / kChunk;
        const uint32_t *h0 = p.hist0 + (int64_t)s * p.nch * 256;
        uint32_t acc = 0;
        for (int c = tid >> 8; c < nch; c += kSelThreads / 256) acc += h0[c * 256 + (tid & 255)];
        atomicAdd(&hist[tid & 255], acc);
        prefix = 0;
        need = p.budget;
    } else {
        if (tid < 256) hist[tid] = p.hist12[((int64_t)s * 2 + (pass - 1)) * 256 + tid];
        const int32_t *st = p.state + ((int64_t)(pass - 1) * S + s) * 2;
        prefix = (uint32_t)st[0];
        need = st[1];
    }
    __syncthreads();
    pick_digit(hist, need, lds_pick);
    if (tid == 0) lds_above = 0u;
    __syncthreads();
    const int pshift = shift + 8;                      // the digit just picked
    prefix |= (uint32_t)lds_pick[0] << pshift;
    need -= lds_pick[1];
    const uint32_t pmask = ~0u << pshift;
    if (blockIdx.x == 0 && tid == 0) {
        int32_t *st = p.state + ((int64_t)pass * S + s) * 2;
        st[0] = (int32_t)prefix;
        st[1] = need;
    }
    __syncthreads();   // lds_pick is read above; hist is reused below
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    uint32_t above = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kSelThreads + tid;
        if (t < t1) {
            if ((key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & 255u], 1u);
            else if (key[u] > prefix) ++above;         // ranks above every key of the prefix
        }
    }
    if (pass == 2) atomicAdd(&lds_above, above);
    __syncthreads();
    if (pass < 2) {
        if (tid < 256 && hist[tid]) atomicAdd(&p.hist12[((int64_t)s * 2 + pass) * 256 + tid], hist[tid]);
    } else {
        uint32_t *lo = p.low + ((int64_t)s * p.nch + blockIdx.x) * 257;
        if (tid < 256) lo[tid] = hist[tid];
        if (tid == 256) lo[256] = lds_above;
    }
}

// Position pass: T and the ties to keep from the summed last-digit
// histograms, the kept and tied counts of the chunks before this one, then the
// chunk's kept positions.
__global__ __launch_bounds__(kSelThreads) void compress_split_write_kernel(CompressParams p) {
    __shared__ uint32_t hist[256];
    __shared__ int lds_pick[2];
    __shared__ uint32_t lds_cnt[2];
    __shared__ int lds_wave[2][kSelWaves];
    const int s = blockIdx.y, tid = threadIdx.x;
    const int S = gridDim.y;
    int n, t0, t1;
    if (!split_chunk(p, &n, &t0, &t1)) return;
    const int nch = (n + kChunk - 1) / kChunk;
    const uint32_t *lo = p.low + (int64_t)s * p.nch * 257;
    const uint32_t *gkeys = p.keys + (int64_t)s * p.key_stride;
    auto load4 = [&](int t) __attribute__((always_inline)) { return *(const u32x4k_t *)(gkeys + t); };
    // the first round's keys are in flight during the sums
    const u32x4k_t k_first = t0 + 4 * tid < t1 ? load4(t0 + 4 * tid) : u32x4k_t{0u, 0u, 0u, 0u};
    if (tid < 256) hist[tid] = 0u;
    if (tid < 2) lds_cnt[tid] = 0u;
    __syncthreads();
    {
        uint32_t acc = 0;
        for (int c = tid >> 8; c < nch; c += kSelThreads / 256) acc += lo[c * 257 + (tid & 255)];
        atomicAdd(&hist[tid & 255], acc);
    }
    const int32_t *st = p.state + ((int64_t)2 * S + s) * 2;
    const uint32_t prefix = (uint32_t)st[0];
    int need = st[1];
    __syncthreads();
    pick_digit(hist, need, lds_pick);
    __syncthreads();
    const uint32_t d = (uint32_t)lds_pick[0];
    const uint32_t T = prefix | d;
    need -= lds_pick[1];   // tokens of key T to keep
    // Keys above T and keys equal to T in the chunks before this one.
    uint32_t gt = 0, eq = 0;
    for (int i = tid; i < (int)blockIdx.x * 257; i += kSelThreads) {
        const int b = i % 257;
        const uint32_t v = lo[i];
        if (b == 256 || (uint32_t)b > d) gt += v;
        else if ((uint32_t)b == d) eq += v;
    }
    if (gt) atomicAdd(&lds_cnt[0], gt);
    if (eq) atomicAdd(&lds_cnt[1], eq);
    __syncthreads();
    const int eq_before = (int)lds_cnt[1];
    const int kept_before = (int)lds_cnt[0] + min(need, eq_before);
    write_kept(load4, t0, t1, T, need, eq_before, kept_before, p.keep + (int64_t)s * p.budget,
               p.budget, lds_wave, k_first);
}

// Moves slice blockIdx.x % slices of kv head blockIdx.x / slices of the kept
// rows of sequence blockIdx.y.  The source and destination slots of a window
// of kept tokens are resolved once into LDS (their keep-list and table loads
// in flight together), so a chunk waits only for its own K/V loads.  With
// near_only set it moves only the kept tokens whose source lies below the
// budget (a prefix of the kept list: sources ascend); the others are left to
// compress_move_far_kernel.
template <bool kScales>
__global__ __launch_bounds__(kMoveThreads) void compress_move_kernel(CompressParams p, int near_only) {
    __shared__ int64_t lds_src[kMoveWindow];   // source slot of kept token w0 + i, or -1 (in place)
    __shared__ int64_t lds_dst[kMoveWindow];
    __shared__ int lds_far[kMoveThreads / 64];
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
        if (near_only && keep[w0] >= budget) break;   // uniform: the rest lie at or past the budget
        constexpr int kPer = kMoveWindow / kMoveThreads;
        int tk[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = u * kMoveThreads + tid;
            tk[u] = i < wn ? keep[w0 + i] : 0;
        }
        int far_first = wn;   // first entry of the window whose source is at or past the budget
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = u * kMoveThreads + tid;
            const int j = w0 + i;
            // kept token tk moves down to j
            const bool mv = i < wn && tk[u] > j && tk[u] < (near_only ? min(n, budget) : n);
            if (i < wn) {
                lds_src[i] = mv ? slot_of(row, tk[u], bs) : -1;
                lds_dst[i] = mv ? slot_of(row, j, bs) : -1;
                if (tk[u] >= budget) far_first = min(far_first, i);
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) far_first = min(far_first, __shfl_xor(far_first, off));
        if ((tid & 63) == 0) lds_far[tid >> 6] = far_first;
        __syncthreads();
        // near_only: sources ascend, so the near tokens are the window's first far_first
        int wn_move = wn;
        if (near_only) {
#pragma unroll
            for (int w = 0; w < kMoveThreads / 64; ++w) wn_move = min(wn_move, lds_far[w]);
        }
        for (int c0 = 0; c0 < wn_move; c0 += kMoveRounds * tok_per_round) {
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

constexpr int kFarWindow = 64;    // kept tokens per workgroup of compress_move_far_kernel

// Moves the kept tokens whose source lies at or past the budget.  Their
// sources are never a destination of this call and the near tokens' sources
// below the budget were read by the launch before, so every such token moves
// independently: workgroup (window, kv head, slice) of sequence blockIdx.y
// moves its window of kFarWindow kept tokens with no ordering at all.
template <bool kScales>
__global__ __launch_bounds__(kMoveThreads) void compress_move_far_kernel(CompressParams p) {
    const int per = p.hkv * p.slices;
    const int win = blockIdx.x / per;
    const int hs = blockIdx.x - win * per;
    const int g = hs / p.slices;
    const int slice = hs - g * p.slices;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int n = p.ctx[s];
    const int budget = p.budget;
    if (n <= budget) return;
    const int j0 = win * kFarWindow;
    if (j0 >= budget) return;
    const int j1 = min(budget, j0 + kFarWindow);
    const int bs = p.block_size;
    const int32_t *row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const int32_t *keep = p.keep + (int64_t)s * budget;
    const int pieces = p.head_bytes / p.slices / 16;
    const int tok_per_round = kMoveThreads / pieces;
    const int piece = tid % pieces;
    const int64_t row_bytes = (int64_t)p.hkv * p.head_bytes;
    const int64_t col = (int64_t)g * p.head_bytes + (int64_t)slice * pieces * 16 + piece * 16;
    char *kbase = (char *)p.k + col;
    char *vbase = (char *)p.v + col;
    const bool lead = slice == 0 && piece == 0;
    for (int c0 = j0; c0 < j1; c0 += kMoveRounds * tok_per_round) {
        u32x4_t kr[kMoveRounds], vr[kMoveRounds];
        float ks[kMoveRounds], vs[kMoveRounds], sc[kMoveRounds];
        int64_t src[kMoveRounds], dst[kMoveRounds];
        int tk[kMoveRounds];
#pragma unroll
        for (int r = 0; r < kMoveRounds; ++r) {
            const int j = c0 + r * tok_per_round + tid / pieces;
            tk[r] = j < j1 ? keep[j] : -1;
        }
#pragma unroll
        for (int r = 0; r < kMoveRounds; ++r) {
            const int j = c0 + r * tok_per_round + tid / pieces;
            const bool mv = tk[r] >= budget && tk[r] < n;
            src[r] = mv ? slot_of(row, tk[r], bs) : -1;
            dst[r] = mv ? slot_of(row, j, bs) : -1;
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

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

size_t r256(int64_t b) { return (size_t)((b + 255) & ~(int64_t)255); }
size_t keep_bytes(int64_t S, int64_t budget) { return r256(S * budget * 4); }
size_t ctx_bytes(int64_t S) { return r256(S * 4); }
int64_t chunks_of(int64_t max_ctx) { return (max_ctx + kChunk - 1) / kChunk; }
// The split select's arrays (keys, first-digit histograms per chunk, digit
// histograms per sequence, states, last-digit histograms per chunk) exist only
// when a context can be longer than the LDS holds.
struct SplitLayout {
    size_t keys, hist0, hist12, state, low, total;
};
SplitLayout split_layout(int64_t S, int64_t max_ctx) {
    SplitLayout l{};
    if (max_ctx <= kLdsKeys) return l;
    const int64_t nch = chunks_of(max_ctx);
    l.keys = 0;
    l.hist0 = l.keys + r256(S * ((max_ctx + 3) & ~(int64_t)3) * 4);
    l.hist12 = l.hist0 + r256(S * nch * 256 * 4);
    l.state = l.hist12 + r256(S * 512 * 4);
    l.low = l.state + r256(3 * S * 2 * 4);
    l.total = l.low + r256(S * nch * 257 * 4);
    return l;
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
    char *split_base = (char *)ws + keep_bytes(sh->num_seqs, budget) + ctx_bytes(sh->num_seqs);
    const SplitLayout sl = split_layout(sh->num_seqs, max_ctx);
    const bool split = max_ctx > kLdsKeys;
    p.keys = (uint32_t *)(split_base + sl.keys);
    p.hist0 = (uint32_t *)(split_base + sl.hist0);
    p.hist12 = (uint32_t *)(split_base + sl.hist12);
    p.state = (int32_t *)(split_base + sl.state);
    p.low = (uint32_t *)(split_base + sl.low);
    p.nch = (int)chunks_of(max_ctx);
    p.key_stride = (int)((max_ctx + 3) & ~(int64_t)3);
    p.hkv = sh->num_kv_heads;
    p.head_bytes = sh->head_dim * elem;
    p.slices = p.head_bytes > kSliceBytes ? p.head_bytes / kSliceBytes : 1;
    p.block_size = sh->block_size;
    p.max_blocks_per_seq = sh->max_blocks_per_seq;
    p.max_ctx = (int)max_ctx;
    p.budget = budget;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (split) {
        const dim3 sgrid((unsigned)p.nch, (unsigned)sh->num_seqs);
        hipLaunchKernelGGL(compress_split_keys_kernel, sgrid, dim3(kSelThreads), 0, st, p);
        for (int shift = 16; shift >= 0; shift -= 8)
            hipLaunchKernelGGL(compress_split_pass_kernel, sgrid, dim3(kSelThreads), 0, st, p, shift);
        hipLaunchKernelGGL(compress_split_write_kernel, sgrid, dim3(kSelThreads), 0, st, p);
    } else {
        hipLaunchKernelGGL(compress_select_kernel, dim3((unsigned)sh->num_seqs), dim3(kSelThreads), 0, st, p);
    }
    const dim3 mgrid((unsigned)(sh->num_kv_heads * p.slices), (unsigned)sh->num_seqs);
    // Long contexts: the kept tokens whose source lies below the budget move in
    // place in order, then all the others at once, spread over windows.
    // Only a sequence longer than the budget has kept tokens, so the windows
    // cover at most min(budget, max_ctx) of them.
    const int64_t wins = (std::min((int64_t)budget, max_ctx) + kFarWindow - 1) / kFarWindow;
    const bool far = split && budget > 0 && wins * sh->num_kv_heads * p.slices < ((int64_t)1 << 31);
    const int near_only = far ? 1 : 0;
    if (int8) hipLaunchKernelGGL(compress_move_kernel<true>, mgrid, dim3(kMoveThreads), 0, st, p, near_only);
    else hipLaunchKernelGGL(compress_move_kernel<false>, mgrid, dim3(kMoveThreads), 0, st, p, near_only);
    if (far) {
        const dim3 fgrid((unsigned)(wins * sh->num_kv_heads * p.slices), (unsigned)sh->num_seqs);
        if (int8) hipLaunchKernelGGL(compress_move_far_kernel<true>, fgrid, dim3(kMoveThreads), 0, st, p);
        else hipLaunchKernelGGL(compress_move_far_kernel<false>, fgrid, dim3(kMoveThreads), 0, st, p);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t paged_kv_compress_workspace_bytes(const pa_score_shape *shape, int32_t budget) {
    if (!shape || shape->num_seqs < 0 || budget < 0) return 0;
    return keep_bytes(shape->num_seqs, budget) + ctx_bytes(shape->num_seqs) +
           split_layout(shape->num_seqs, (int64_t)shape->max_blocks_per_seq * shape->block_size).total;
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
