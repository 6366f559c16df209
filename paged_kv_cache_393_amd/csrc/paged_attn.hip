// paged_attn.hip -- PagedAttention decode for gfx950 (CDNA4) behind the C-ABI
// of include/paged_attn.h.
//
// What is computed: for each sequence s and query head h, the decode query
// attends over the sequence's context gathered through its block table, with
// G = Hq / Hkv consecutive query heads sharing kv head h / G, scores
// scale * q.k and one exact softmax over the whole context (ybb.press page
// "LLM 推理 KV Cache 内存管理深度工程实践", sections 2.2 and 6.2; t6page
// "KV cache" page, section "PagedAttention 的算子").  The int8 variant
// dequantizes code * per-(slot, kv head) scale (same ybb.press page, 6.1).
//
// Work decomposition.  One workgroup (4 waves) owns one context partition of
// one (sequence, kv head, chunk of <= 16 query heads of the group).  Inside
// it the 16-token tiles of the partition are dealt round-robin to the waves;
// each wave keeps its own online-softmax state and the four are merged in
// LDS at the end.  With several partitions per sequence each workgroup writes
// an unnormalised partial (acc, max, sum) and a reduction kernel merges them
// (log-sum-exp weights, fixed partition order, so results are reproducible).
//
// Per tile and wave:
//   * K: lane l loads 16 B of token l%16 (dims chosen so that the four lane
//     groups cover complementary dims) -> the A operand of
//     v_mfma_f32_16x16x16_bf16 with tokens as rows; the group's query heads
//     (zero-padded to 16) are the B operand, loaded once.  The MFMA result
//     gives lane l the scores of head l%16 for tokens 4*(l/16)..+3.
//   * softmax: tile max over the 16 tokens (two xor-shuffles), running max and
//     rescale factor, p = 2^(s*scale*log2e - m); p and the rescale factor go to
//     a per-wave LDS slot.
//   * V: lane l loads 16 B (8 dims) of one token per load, fully coalesced
//     (head_dim/8 lanes per token row), converts to fp32 and accumulates
//     p * v for every head of the chunk with fp32 FMAs (fp32 P, no bf16
//     rounding of probabilities).
//   * the next tile's K/V loads are issued before the current tile is
//     processed (register double buffering).
// Tokens past the context end inside the last tile are never loaded: their
// loads are clamped to the last valid token and their scores set to -inf, so
// their weight is exactly 0 and padding contents cannot reach the output.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTile = 16;           // tokens per tile (MFMA rows)
constexpr int kWaves = 4;           // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxChunkHeads = 16;  // query heads per workgroup (MFMA columns)
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeParams {
    const uint16_t *q;       // bf16 [S, Hq, D]
    const void *k;           // [NB, bs, Hkv, D] bf16 or int8
    const void *v;
    const float *k_scales;   // [NB, bs, Hkv] (int8 only)
    const float *v_scales;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *out;              // fp32 [S, Hq, D]
    float *part_acc;         // fp32 [S, Hq, P, D]      (P > 1 only)
    float *part_ml;          // fp32 [S, Hq, P, 2]
    float scale_log2;        // softmax scale * log2(e)
    int num_q_heads;
    int num_kv_heads;
    int group;               // Hq / Hkv
    int n_chunks;            // ceil(group / chunk heads)
    int max_blocks_per_seq;
    int log2_block_size;
    int split_tokens;        // multiple of kTile
    int max_splits;
};

struct ReduceParams {
    const int32_t *context_lens;
    const float *part_acc;
    const float *part_ml;
    float *out;
    int num_q_heads;
    int split_tokens;
    int max_splits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four signed bytes -> four bf16 (exact: |code| <= 128 has at most 8 significant bits).
__device__ __forceinline__ bf16x4_t i8x4_to_bf16x4(uint32_t w) {
    float f0 = (float)(int)(int8_t)(w & 0xffu);
    float f1 = (float)(int)(int8_t)((w >> 8) & 0xffu);
    float f2 = (float)(int)(int8_t)((w >> 16) & 0xffu);
    float f3 = (float)(int)(int8_t)(w >> 24);
    u32x2_t r;
    r.x = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
    r.y = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
    return __builtin_bit_cast(bf16x4_t, r);
}

__device__ __forceinline__ float i8_at(uint32_t w, int b) {
    return (float)(int)(int8_t)((w >> (8 * b)) & 0xffu);
}

// Order this wave's LDS writes before its following LDS reads (other lanes'
// data); LDS requests of one wave complete in order.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, bool INT8>
struct Layout {
    static constexpr int kElem = INT8 ? 1 : 2;                 // bytes per cache element
    static constexpr int kKElemsPerLoad = 16 / kElem;          // K dims per 16-B load
    static constexpr int kKLoads = D / (4 * kKElemsPerLoad);   // 16-B K loads per lane per tile
    static constexpr int kSteps = D / 16;                      // MFMA k-steps (4 dims x 4 groups)
    static constexpr int kStepsPerLoad = kKElemsPerLoad / 4;
    static constexpr int kLanesPerRow = D / 8;                 // V: 8 dims per lane
    static constexpr int kRows = 64 / kLanesPerRow;            // V tokens per load instruction
    static constexpr int kVLoads = kTile / kRows;              // V loads per lane per tile
    using VReg = typename std::conditional<INT8, u32x2_t, u32x4_t>::type;
    // First dim of MFMA step `st` for lane group `lg`; the step covers 4 dims.
    __device__ static constexpr int step_dim(int st, int lg) {
        return (st / kStepsPerLoad) * 4 * kKElemsPerLoad + kKElemsPerLoad * lg +
               4 * (st % kStepsPerLoad);
    }
};

template <int D, bool INT8>
struct TileRegs {
    using L = Layout<D, INT8>;
    u32x4_t k[L::kKLoads];
    typename L::VReg v[L::kVLoads];
    float sc;   // int8: lanes 0..15 K scale of token lane, 16..31 V scale of token lane-16
};

template <int D, int GT, bool INT8>
__global__ __launch_bounds__(kThreads) void pa_decode_kernel(const DecodeParams p) {
    using L = Layout<D, INT8>;
    static_assert(GT >= 1 && GT <= kMaxChunkHeads, "chunk heads");
    static_assert(L::kKLoads >= 1 && L::kVLoads >= 1, "head_dim");

    __shared__ __attribute__((aligned(16))) float lds_p[kWaves][GT][kTile];
    __shared__ float lds_alpha[kWaves][GT];
    __shared__ __attribute__((aligned(16))) float lds_sc[kWaves][2 * kTile];
    __shared__ float lds_acc[kWaves][GT][D];
    __shared__ float lds_m[kWaves][GT];
    __shared__ float lds_l[kWaves][GT];

    const int split = blockIdx.x;
    const int g = blockIdx.y / p.n_chunks;
    const int chunk = blockIdx.y - g * p.n_chunks;
    const int s = blockIdx.z;
    const int ctx = p.context_lens[s];
    const int t_begin = split * p.split_tokens;
    const bool single = p.max_splits == 1;
    if (!single && t_begin >= ctx) return;   // empty partition; the reduction skips it
    const int t_end = min(ctx, t_begin + p.split_tokens);
    const int n_tiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

    const int Hq = p.num_q_heads;
    const int h_base = g * p.group + chunk * GT;
    const int n_heads = min(GT, p.group - chunk * GT);

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4;      // lane group (MFMA k group / score rows)
    const int l16 = lane & 15;     // token row of K, head column of Q and scores
    const int vr = lane / L::kLanesPerRow;   // V token row
    const int vc = lane % L::kLanesPerRow;   // V 8-dim column

    const int bs_log2 = p.log2_block_size;
    const int bs_mask = (1 << bs_log2) - 1;
    const int64_t row_bytes = (int64_t)p.num_kv_heads * D * L::kElem;   // one token slot
    const char *kbase = (const char *)p.k + (int64_t)g * D * L::kElem;
    const char *vbase = (const char *)p.v + (int64_t)g * D * L::kElem;
    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;

    // Query operand (B of the MFMA): head l16 of the chunk, zero for padding heads.
    bf16x4_t qop[L::kSteps];
    {
        const bool live = l16 < n_heads;
        const uint16_t *qrow = p.q + ((int64_t)s * Hq + h_base + (live ? l16 : 0)) * D;
#pragma unroll
        for (int st = 0; st < L::kSteps; ++st) {
            u32x2_t w = *(const u32x2_t *)(qrow + L::step_dim(st, lg));
            if (!live) w = u32x2_t{0u, 0u};
            qop[st] = __builtin_bit_cast(bf16x4_t, w);
        }
    }

    // Block-table entries of this partition, 64 at a time: lane i holds entry tbl_base + i.
    const int blk_first = t_begin >> bs_log2;
    const int blk_last = t_end > t_begin ? ((t_end - 1) >> bs_log2) + 1 : blk_first;
    int tbl_base = blk_first;
    int tbl_val = (blk_first + lane < blk_last) ? table[blk_first + lane] : 0;

    // Token-slot index phys * block_size + slot of the first token of tile `tile`.
    auto tile_slot = [&](int tile) -> int64_t {
        const int t0 = t_begin + tile * kTile;
        const int blk = t0 >> bs_log2;
        if (blk - tbl_base >= 64) {          // wave-uniform: refill the table window
            tbl_base = blk;
            tbl_val = (blk + lane < blk_last) ? table[blk + lane] : 0;
        }
        const int phys = __builtin_amdgcn_readlane(tbl_val, blk - tbl_base);
        return ((int64_t)phys << bs_log2) + (t0 & bs_mask);
    };

    auto load_tile = [&](TileRegs<D, INT8> &r, int tile) {
        const int t0 = t_begin + tile * kTile;
        const int last = t_end - 1 - t0;                 // last valid row of this tile
        const int64_t slot0 = tile_slot(tile);
        const int64_t off = slot0 * row_bytes;
        const int kt = min(l16, last);
        const char *kp = kbase + off + kt * row_bytes;
#pragma unroll
        for (int m = 0; m < L::kKLoads; ++m)
            r.k[m] = *(const u32x4_t *)(kp + (L::step_dim(m * L::kStepsPerLoad, lg)) * L::kElem);
#pragma unroll
        for (int j = 0; j < L::kVLoads; ++j) {
            const int vt = min(vr * L::kVLoads + j, last);
            r.v[j] = *(const typename L::VReg *)(vbase + off + vt * row_bytes +
                                                 vc * 8 * L::kElem);
        }
        if constexpr (INT8) {
            const int st = min(l16, last);
            const int64_t slot = slot0 + st;
            const float *sp = (lane & 16) ? p.v_scales : p.k_scales;
            r.sc = sp[slot * p.num_kv_heads + g];
        }
    };

    // Online-softmax state of this wave.  Score lanes: head l16, rows 4*lg..4*lg+3.
    float m_run = -INFINITY;
    float l_run = 0.f;
    float acc[GT][8];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    auto compute_tile = [&](const TileRegs<D, INT8> &r, int tile) {
        const int t0 = t_begin + tile * kTile;
        wave_lds_sync();
        if constexpr (INT8) {
            if (lane < 2 * kTile) lds_sc[wave][lane] = r.sc;
        }
        // S = K Q^T on the matrix cores: rows = tokens, columns = heads.
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < L::kSteps; ++st) {
            const int m = st / L::kStepsPerLoad;
            const int sub = st % L::kStepsPerLoad;
            bf16x4_t a;
            if constexpr (INT8) {
                a = i8x4_to_bf16x4(r.k[m][sub]);
            } else {
                u32x2_t w = sub == 0 ? u32x2_t{r.k[m].x, r.k[m].y} : u32x2_t{r.k[m].z, r.k[m].w};
                a = __builtin_bit_cast(bf16x4_t, w);
            }
            sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, qop[st], sacc, 0, 0, 0);
        }
        float ks[4] = {1.f, 1.f, 1.f, 1.f}, vsc[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (INT8) {
            wave_lds_sync();
            f32x4_t kv4 = *(const f32x4_t *)&lds_sc[wave][4 * lg];
            f32x4_t vv4 = *(const f32x4_t *)&lds_sc[wave][kTile + 4 * lg];
            ks[0] = kv4.x; ks[1] = kv4.y; ks[2] = kv4.z; ks[3] = kv4.w;
            vsc[0] = vv4.x; vsc[1] = vv4.y; vsc[2] = vv4.z; vsc[3] = vv4.w;
        }
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = sacc[i] * (INT8 ? p.scale_log2 * ks[i] : p.scale_log2);
            sc[i] = (t0 + 4 * lg + i < t_end) ? x : -INFINITY;
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);              // finite: a tile has a valid token
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float pr[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
            psum += pr[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (l16 < GT) {
            f32x4_t pw = {pr[0] * vsc[0], pr[1] * vsc[1], pr[2] * vsc[2], pr[3] * vsc[3]};
            *(f32x4_t *)&lds_p[wave][l16][4 * lg] = pw;
            if (lg == 0) lds_alpha[wave][l16] = alpha;
        }
        wave_lds_sync();
        // O += P V with fp32 FMAs; this lane owns dims 8*vc..8*vc+7 of token rows vr*kVLoads+j.
        float vf[L::kVLoads][8];
#pragma unroll
        for (int j = 0; j < L::kVLoads; ++j) {
            if constexpr (INT8) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    vf[j][b] = i8_at(r.v[j].x, b);
                    vf[j][4 + b] = i8_at(r.v[j].y, b);
                }
            } else {
                vf[j][0] = bf16_lo(r.v[j].x); vf[j][1] = bf16_hi(r.v[j].x);
                vf[j][2] = bf16_lo(r.v[j].y); vf[j][3] = bf16_hi(r.v[j].y);
                vf[j][4] = bf16_lo(r.v[j].z); vf[j][5] = bf16_hi(r.v[j].z);
                vf[j][6] = bf16_lo(r.v[j].w); vf[j][7] = bf16_hi(r.v[j].w);
            }
        }
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            const float a = lds_alpha[wave][h];
            float pw[L::kVLoads];
#pragma unroll
            for (int j = 0; j < L::kVLoads; ++j) pw[j] = lds_p[wave][h][vr * L::kVLoads + j];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = acc[h][e] * a;
#pragma unroll
                for (int j = 0; j < L::kVLoads; ++j) x = fmaf(pw[j], vf[j][e], x);
                acc[h][e] = x;
            }
        }
    };

    if (wave < n_tiles) {
        TileRegs<D, INT8> ra, rb;
        int tile = wave;
        load_tile(ra, tile);
        for (;;) {
            const int t1 = tile + kWaves;
            const bool more1 = t1 < n_tiles;
            load_tile(rb, more1 ? t1 : tile);      // unconditional: keeps the loads in flight
            compute_tile(ra, tile);
            if (!more1) break;
            const int t2 = t1 + kWaves;
            const bool more2 = t2 < n_tiles;
            load_tile(ra, more2 ? t2 : t1);
            compute_tile(rb, t1);
            if (!more2) break;
            tile = t2;
        }
    }

    // Merge inside the wave: the four score-lane groups hold partial sums, the
    // V token rows hold partial accumulators over different tokens.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
#pragma unroll
    for (int off = L::kLanesPerRow; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    if (lane < GT) {
        lds_m[wave][lane] = m_run;
        lds_l[wave][lane] = l_run;
    }
    if (vr == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) lds_acc[wave][h][vc * 8 + e] = acc[h][e];
    }
    __syncthreads();

    // Merge across waves and write the result (or this partition's partial).
    for (int idx = threadIdx.x; idx < GT * D; idx += kThreads) {
        const int h = idx / D;
        const int d = idx - h * D;
        if (h >= n_heads) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][h]);
        float Lsum = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = lds_m[w][h];
            const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            Lsum = fmaf(f, lds_l[w][h], Lsum);
            A = fmaf(f, lds_acc[w][h][d], A);
        }
        const int64_t row = (int64_t)s * Hq + h_base + h;
        if (single) {
            p.out[row * D + d] = Lsum > 0.f ? A / Lsum : 0.f;
        } else {
            const int64_t pr = row * p.max_splits + split;
            p.part_acc[pr * D + d] = A;
            if (d == 0) {
                p.part_ml[2 * pr] = M;
                p.part_ml[2 * pr + 1] = Lsum;
            }
        }
    }
}

// Merge the partitions of one (sequence, query head): weights 2^(m_p - M) l_p,
// partitions visited in index order.
template <int D>
__global__ __launch_bounds__(64) void pa_reduce_kernel(const ReduceParams p) {
    constexpr int kPer = D / 64;
    const int row = blockIdx.x;                 // s * Hq + h
    const int s = row / p.num_q_heads;
    const int lane = threadIdx.x;
    const int ctx = p.context_lens[s];
    const int n = (ctx + p.split_tokens - 1) / p.split_tokens;
    const float *ml = p.part_ml + (int64_t)row * p.max_splits * 2;
    const float *pa = p.part_acc + (int64_t)row * p.max_splits * D;
    float M = -INFINITY;
    for (int i = 0; i < n; ++i) M = fmaxf(M, ml[2 * i]);
    float Lsum = 0.f;
    float A[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) A[e] = 0.f;
    for (int i = 0; i < n; ++i) {
        const float f = __builtin_amdgcn_exp2f(ml[2 * i] - M);
        Lsum = fmaf(f, ml[2 * i + 1], Lsum);
#pragma unroll
        for (int e = 0; e < kPer; ++e) A[e] = fmaf(f, pa[(int64_t)i * D + lane * kPer + e], A[e]);
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e)
        p.out[(int64_t)row * D + lane * kPer + e] = Lsum > 0.f ? A[e] / Lsum : 0.f;
}

// ----------------------------------------------------------------------------
// Host side: validation, plan, dispatch.

struct Plan {
    int split_tokens;
    int max_splits;
    int chunk_heads;   // template GT
    int n_chunks;
    int log2_bs;
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

int make_plan(const pa_shape *sh, Plan *pl) {
    if (!sh) return PA_ERR_NULL;
    if (sh->num_seqs < 0 || sh->num_q_heads <= 0 || sh->num_kv_heads <= 0 ||
        sh->head_dim <= 0 || sh->block_size <= 0 || sh->max_blocks_per_seq <= 0 ||
        sh->num_blocks <= 0 || sh->split_tokens < 0)
        return PA_ERR_SHAPE;
    if (sh->num_q_heads % sh->num_kv_heads != 0) return PA_ERR_SHAPE;
    if (sh->head_dim != 64 && sh->head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(sh->block_size) || sh->block_size < kTile || sh->block_size > 4096)
        return PA_ERR_UNSUPPORTED;
    if (sh->split_tokens % kTile != 0) return PA_ERR_SHAPE;
    const int64_t max_ctx = (int64_t)sh->max_blocks_per_seq * sh->block_size;
    if (max_ctx > (int64_t)1 << 30) return PA_ERR_SHAPE;
    const int group = sh->num_q_heads / sh->num_kv_heads;
    int gt = 1;
    while (gt < group && gt < kMaxChunkHeads) gt <<= 1;
    pl->chunk_heads = gt;
    pl->n_chunks = (group + gt - 1) / gt;
    pl->log2_bs = ilog2(sh->block_size);
    int T = sh->split_tokens;
    if (T == 0) T = 512;            // default partition; one partition if the context is shorter
    if ((int64_t)T >= max_ctx) {
        pl->split_tokens = (int)((max_ctx + kTile - 1) / kTile * kTile);
        pl->max_splits = 1;
    } else {
        pl->split_tokens = T;
        pl->max_splits = (int)((max_ctx + T - 1) / T);
    }
    if ((int64_t)sh->num_kv_heads * pl->n_chunks > 65535 || sh->num_seqs > 65535)
        return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

size_t workspace_for(const pa_shape *sh, const Plan &pl) {
    if (pl.max_splits <= 1) return 0;
    const size_t rows = (size_t)sh->num_seqs * sh->num_q_heads * pl.max_splits;
    const size_t acc = (rows * sh->head_dim * sizeof(float) + 255) & ~(size_t)255;
    return acc + rows * 2 * sizeof(float);
}

template <int D, bool INT8>
int launch_decode_d(const DecodeParams &prm, const Plan &pl, int S, int Hkv, hipStream_t st) {
    dim3 grid(pl.max_splits, Hkv * pl.n_chunks, S);
    dim3 block(kThreads);
    switch (pl.chunk_heads) {
        case 1: hipLaunchKernelGGL((pa_decode_kernel<D, 1, INT8>), grid, block, 0, st, prm); break;
        case 2: hipLaunchKernelGGL((pa_decode_kernel<D, 2, INT8>), grid, block, 0, st, prm); break;
        case 4: hipLaunchKernelGGL((pa_decode_kernel<D, 4, INT8>), grid, block, 0, st, prm); break;
        case 8: hipLaunchKernelGGL((pa_decode_kernel<D, 8, INT8>), grid, block, 0, st, prm); break;
        case 16: hipLaunchKernelGGL((pa_decode_kernel<D, 16, INT8>), grid, block, 0, st, prm); break;
        default: return PA_ERR_UNSUPPORTED;
    }
    if (pl.max_splits > 1) {
        ReduceParams rp;
        rp.context_lens = prm.context_lens;
        rp.part_acc = prm.part_acc;
        rp.part_ml = prm.part_ml;
        rp.out = prm.out;
        rp.num_q_heads = prm.num_q_heads;
        rp.split_tokens = pl.split_tokens;
        rp.max_splits = pl.max_splits;
        hipLaunchKernelGGL((pa_reduce_kernel<D>), dim3(S * prm.num_q_heads), dim3(64), 0, st, rp);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int decode_common(bool int8, const void *q, const void *k, const void *v, const float *ks,
                  const float *vs, const int32_t *bt, const int32_t *cl, float scale, float *out,
                  const pa_shape *sh, void *ws, size_t ws_bytes, void *stream) {
    Plan pl;
    int rc = make_plan(sh, &pl);
    if (rc != PA_OK) return rc;
    if (sh->num_seqs == 0) return PA_OK;
    if (!q || !k || !v || !bt || !cl || !out) return PA_ERR_NULL;
    if (int8 && (!ks || !vs)) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PA_ERR_ALIGNMENT;
    const size_t need = workspace_for(sh, pl);
    if (need > 0 && (!ws || ws_bytes < need)) return PA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return PA_ERR_ALIGNMENT;

    DecodeParams prm;
    prm.q = (const uint16_t *)q;
    prm.k = k;
    prm.v = v;
    prm.k_scales = ks;
    prm.v_scales = vs;
    prm.block_tables = bt;
    prm.context_lens = cl;
    prm.out = out;
    const size_t rows = (size_t)sh->num_seqs * sh->num_q_heads * pl.max_splits;
    const size_t acc_bytes = (rows * sh->head_dim * sizeof(float) + 255) & ~(size_t)255;
    prm.part_acc = need ? (float *)ws : nullptr;
    prm.part_ml = need ? (float *)((char *)ws + acc_bytes) : nullptr;
    prm.scale_log2 = scale * kLog2e;
    prm.num_q_heads = sh->num_q_heads;
    prm.num_kv_heads = sh->num_kv_heads;
    prm.group = sh->num_q_heads / sh->num_kv_heads;
    prm.n_chunks = pl.n_chunks;
    prm.max_blocks_per_seq = sh->max_blocks_per_seq;
    prm.log2_block_size = pl.log2_bs;
    prm.split_tokens = pl.split_tokens;
    prm.max_splits = pl.max_splits;
    hipStream_t st = (hipStream_t)stream;
    if (sh->head_dim == 128)
        return int8 ? launch_decode_d<128, true>(prm, pl, sh->num_seqs, sh->num_kv_heads, st)
                    : launch_decode_d<128, false>(prm, pl, sh->num_seqs, sh->num_kv_heads, st);
    return int8 ? launch_decode_d<64, true>(prm, pl, sh->num_seqs, sh->num_kv_heads, st)
                : launch_decode_d<64, false>(prm, pl, sh->num_seqs, sh->num_kv_heads, st);
}

}  // namespace

extern "C" {

int paged_attn_plan(const pa_shape *shape, int32_t *split_tokens, int32_t *max_splits) {
    Plan pl;
    int rc = make_plan(shape, &pl);
    if (rc != PA_OK) return rc;
    if (split_tokens) *split_tokens = pl.split_tokens;
    if (max_splits) *max_splits = pl.max_splits;
    return PA_OK;
}

size_t paged_attn_workspace_bytes(const pa_shape *shape) {
    Plan pl;
    if (make_plan(shape, &pl) != PA_OK) return 0;
    return workspace_for(shape, pl);
}

int paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      float *out, const pa_shape *shape, void *workspace, size_t workspace_bytes,
                      void *stream) {
    return decode_common(false, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                         scale, out, shape, workspace, workspace_bytes, stream);
}

int paged_attn_decode_int8(const void *q, const int8_t *k_cache, const int8_t *v_cache,
                           const float *k_scales, const float *v_scales,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           float *out, const pa_shape *shape, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return decode_common(true, q, k_cache, v_cache, k_scales, v_scales, block_tables,
                         context_lens, scale, out, shape, workspace, workspace_bytes, stream);
}

const char *paged_attn_strerror(int code) {
    switch (code) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "invalid shape";
        case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size or grid size";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        case PA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        default: return "unknown error";
    }
}

int paged_attn_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
