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
// Work decomposition.  One wave owns one (sequence, kv head, chunk of <= 16
// query heads of the group, context partition) and streams the partition's
// 16-token tiles with a private online-softmax state; a workgroup holds four
// such waves for four kv heads of the same (sequence, partition), so the
// token rows of a block (all kv heads side by side) are read together.  With
// several partitions per sequence each wave writes an unnormalised partial
// (acc, max, sum) and a reduction kernel merges them (log-sum-exp weights,
// fixed partition order, so results are reproducible).
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
// Rows of the last tile past the context end are slots of the same allocated
// block; they are loaded with the tile but selected away (score -inf, V and
// int8 V scale replaced by 0), so padding contents cannot reach the output.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

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
constexpr int kMaxPartitionBlocks = 64;    // blocks one partition may span (one wave of ids)
constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw (unformatted, stride 0) buffer resource on CDNA3/CDNA4.
constexpr int kRsrcFlags = 0x00020000;

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
    float ks;   // int8: K scale of token row l%16 (every lane group holds the same)
    float vs;   // int8: V scale of token row l%16
};

template <int D, int GT, bool INT8>
__global__ __launch_bounds__(kThreads) void pa_decode_kernel(const DecodeParams p) {
    using L = Layout<D, INT8>;
    static_assert(GT >= 1 && GT <= kMaxChunkHeads, "chunk heads");
    static_assert(L::kKLoads >= 1 && L::kVLoads >= 1, "head_dim");

    __shared__ __attribute__((aligned(16))) float lds_p[kWaves][GT][kTile];
    __shared__ float lds_alpha[kWaves][GT];
    __shared__ __attribute__((aligned(16))) float lds_sc[kWaves][2 * kTile];
    __shared__ float lds_ml[kWaves][2][GT];

    // Grid: x = group of kWaves (kv head, head chunk) units, y = partition,
    // z = sequence.  Each wave owns one unit and streams the whole partition,
    // so the waves of a workgroup read the same blocks' token rows (their kv
    // heads side by side) at about the same time.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
    const int unit = blockIdx.x * kWaves + wave;
    const int Hkv = p.num_kv_heads;
    if (unit >= Hkv * p.n_chunks) return;            // whole wave; no workgroup barrier follows
    const int g = unit / p.n_chunks;
    const int chunk = unit - g * p.n_chunks;
    const int split = blockIdx.y;
    const int s = blockIdx.z;
    const int ctx = p.context_lens[s];
    const int t_begin = split * p.split_tokens;
    const bool single = p.max_splits == 1;
    if (!single && t_begin >= ctx) return;           // empty partition; the reduction skips it
    const int t_end = min(ctx, t_begin + p.split_tokens);
    const int n_tiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

    const int Hq = p.num_q_heads;
    const int h_base = g * p.group + chunk * GT;
    const int n_heads = min(GT, p.group - chunk * GT);

    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4;      // lane group (MFMA k group / score rows)
    const int l16 = lane & 15;     // token row of K, head column of Q and scores
    const int vr = lane / L::kLanesPerRow;   // V token row
    const int vc = lane % L::kLanesPerRow;   // V 8-dim column

    const int bs_log2 = p.log2_block_size;
    const int bs_mask = (1 << bs_log2) - 1;
    const int64_t row_bytes = (int64_t)Hkv * D * L::kElem;   // one token slot, all kv heads
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

    // Block ids of this partition as a register window: lane i holds table
    // entry blk_first + i (a partition spans at most 64 blocks), loaded once
    // before the tile loop; a tile's id is then read with readlane, so the loop
    // itself makes no dependent memory access.
    const int blk_first = t_begin >> bs_log2;
    const int blk_last = t_end > t_begin ? ((t_end - 1) >> bs_log2) + 1 : blk_first;
    const int win = (lane < blk_last - blk_first) ? table[blk_first + lane] : 0;

    // Token-slot index phys * block_size + slot of the first token of tile `tile` (uniform).
    auto tile_slot = [&](int tile) __attribute__((always_inline)) -> int64_t {
        const int t0 = t_begin + tile * kTile;
        const int phys = __builtin_amdgcn_readlane(win, (t0 >> bs_log2) - blk_first);
        return ((int64_t)phys << bs_log2) + (t0 & bs_mask);
    };

    // Tile loads are raw buffer loads: a uniform buffer resource per tile whose
    // range is the tile's valid rows, plus per-lane byte offsets that are fixed
    // for the whole loop -- no per-tile vector address arithmetic.  A tile never
    // crosses a block (block_size is a multiple of 16).  Rows at or past the
    // context end fall outside the resource's range: the hardware returns 0 for
    // them without touching memory, and they are also selected away below
    // (score -inf, V and int8 V scale 0), so padding cannot reach the output.
    const uint32_t rb32 = (uint32_t)row_bytes;
    const int k_off = (int)((uint32_t)l16 * rb32 + (uint32_t)(L::step_dim(0, lg) * L::kElem));
    int v_off[L::kVLoads];
#pragma unroll
    for (int j = 0; j < L::kVLoads; ++j)
        v_off[j] = (int)((uint32_t)(vr * L::kVLoads + j) * rb32 + (uint32_t)(vc * 8 * L::kElem));
    const int s_off = (int)(((uint32_t)l16 * (uint32_t)Hkv + (uint32_t)g) * 4u);

    auto load_tile = [&](TileRegs<D, INT8> &r, int tile) __attribute__((always_inline)) {
        const int64_t slot0 = tile_slot(tile);
        const int rows = min(kTile, t_end - (t_begin + tile * kTile));
        const int range = rows * (int)rb32;
        const __amdgpu_buffer_rsrc_t kr =
            __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + slot0 * row_bytes), 0, range, kRsrcFlags);
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + slot0 * row_bytes), 0, range, kRsrcFlags);
#pragma unroll
        for (int m = 0; m < L::kKLoads; ++m)
            r.k[m] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         kr, k_off + m * 4 * L::kKElemsPerLoad * L::kElem, 0, 0));
#pragma unroll
        for (int j = 0; j < L::kVLoads; ++j) {
            if constexpr (INT8)
                r.v[j] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(vrs, v_off[j], 0, 0));
            else
                r.v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, v_off[j], 0, 0));
        }
        if constexpr (INT8) {
            const int srange = rows * Hkv * 4;
            const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.k_scales + slot0 * Hkv), 0, srange, kRsrcFlags);
            const __amdgpu_buffer_rsrc_t vsr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.v_scales + slot0 * Hkv), 0, srange, kRsrcFlags);
            r.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksr, s_off, 0, 0));
            r.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsr, s_off, 0, 0));
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

    auto compute_tile = [&](const TileRegs<D, INT8> &r, int tile) __attribute__((always_inline)) {
        const int t0 = t_begin + tile * kTile;
        wave_lds_sync();
        if constexpr (INT8) {
            if (lane < kTile) lds_sc[wave][lane] = r.ks;
            else if (lane < 2 * kTile) lds_sc[wave][lane] = r.vs;
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
            // Masked rows: p is exactly 0, and an int8 V scale there may be anything.
            f32x4_t pw;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pw[i] = INT8 ? (sc[i] == -INFINITY ? 0.f : pr[i] * vsc[i]) : pr[i];
            *(f32x4_t *)&lds_p[wave][l16][4 * lg] = pw;
            if (lg == 0) lds_alpha[wave][l16] = alpha;
        }
        wave_lds_sync();
        // O += P V with fp32 FMAs; this lane owns dims 8*vc..8*vc+7 of token rows vr*kVLoads+j.
        float pw[GT][L::kVLoads];
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            const float a = lds_alpha[wave][h];
#pragma unroll
            for (int j = 0; j < L::kVLoads; ++j) pw[h][j] = lds_p[wave][h][vr * L::kVLoads + j];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= a;
        }
        // Rows past the context end (last tile only) are replaced by zeros.
        const int last_row = t_end - 1 - t0;                 // uniform
        const bool partial = last_row < kTile - 1;
#pragma unroll
        for (int j = 0; j < L::kVLoads; ++j) {
            typename L::VReg vr_j = r.v[j];
            if (partial && vr * L::kVLoads + j > last_row) vr_j = typename L::VReg{};
            float vf[8];
            if constexpr (INT8) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    vf[b] = i8_at(vr_j.x, b);
                    vf[4 + b] = i8_at(vr_j.y, b);
                }
            } else {
                vf[0] = bf16_lo(vr_j.x); vf[1] = bf16_hi(vr_j.x);
                vf[2] = bf16_lo(vr_j.y); vf[3] = bf16_hi(vr_j.y);
                vf[4] = bf16_lo(vr_j.z); vf[5] = bf16_hi(vr_j.z);
                vf[6] = bf16_lo(vr_j.w); vf[7] = bf16_hi(vr_j.w);
            }
#pragma unroll
            for (int h = 0; h < GT; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pw[h][j], vf[e], acc[h][e]);
        }
    };

    // Register pipeline of kStages tile buffers: while the wave processes one
    // tile, the loads of its next kStages-1 tiles are in flight.  The scheduling
    // barriers keep each prefetch issued before the processing of the current
    // tile starts.  The loop runs whole rounds of kStages tiles (one back edge,
    // no early exit), so the set of pending loads at its head is the same on
    // entry and on every iteration; the last 0..kStages-1 tiles, already in
    // flight, are processed after it.  Prefetches past the end re-load the last
    // tile (a cache hit), which keeps every load unconditional.
    constexpr int kStages = 3;
    if (n_tiles > 0) {
        TileRegs<D, INT8> buf[kStages];
        auto tile_of = [&](int k) __attribute__((always_inline)) { return min(k, n_tiles - 1); };
        // One pipeline step on buffer I (a compile-time index): prefetch tile
        // k + kStages - 1 into the buffer freed by the previous step, then
        // process tile k.
        auto step = [&](auto I, int k) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            load_tile(buf[(i + kStages - 1) % kStages], tile_of(k + kStages - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute_tile(buf[i], k);
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        static_assert(kStages == 3, "three explicit steps below");
        load_tile(buf[0], tile_of(0));
        __builtin_amdgcn_sched_barrier(0);
        load_tile(buf[1], tile_of(1));
        __builtin_amdgcn_sched_barrier(0);
        const int rounds = n_tiles / kStages;
        for (int rd = 0; rd < rounds; ++rd) {
            step(I0{}, rd * kStages);
            step(I1{}, rd * kStages + 1);
            step(I2{}, rd * kStages + 2);
        }
        const int rem = n_tiles - rounds * kStages;
        if (rem > 0) compute_tile(buf[0], rounds * kStages);
        if (rem > 1) compute_tile(buf[1], rounds * kStages + 1);
    }

    // Finish inside the wave: the four score-lane groups hold partial sums, the
    // V token rows hold partial accumulators over different tokens.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
#pragma unroll
    for (int off = L::kLanesPerRow; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    wave_lds_sync();
    if (lane < GT) {
        lds_ml[wave][0][lane] = m_run;
        lds_ml[wave][1][lane] = l_run;
    }
    wave_lds_sync();
    if (vr == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            if (h >= n_heads) continue;                      // uniform; keeps the loop unrollable
            const int64_t row = (int64_t)s * Hq + h_base + h;
            const float lsum = lds_ml[wave][1][h];
            f32x4_t o0, o1;
            if (single) {
                const float inv = lsum > 0.f ? 1.f / lsum : 0.f;   // lsum == 0 only for ctx == 0
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o0[e] = acc[h][e] * inv;
                    o1[e] = acc[h][4 + e] * inv;
                }
                float *dst = p.out + row * D + vc * 8;
                *(f32x4_t *)dst = o0;
                *(f32x4_t *)(dst + 4) = o1;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o0[e] = acc[h][e];
                    o1[e] = acc[h][4 + e];
                }
                const int64_t pr = row * p.max_splits + split;
                float *dst = p.part_acc + pr * D + vc * 8;
                *(f32x4_t *)dst = o0;
                *(f32x4_t *)(dst + 4) = o1;
                if (vc == 0) {
                    p.part_ml[2 * pr] = lds_ml[wave][0][h];
                    p.part_ml[2 * pr + 1] = lsum;
                }
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
    // A partition may span at most kMaxPartitionBlocks blocks (its ids fit one wave).
    const int64_t t_cap = (int64_t)(kMaxPartitionBlocks - 1) * sh->block_size / kTile * kTile;
    if (T > t_cap) T = (int)t_cap;
    if ((int64_t)T >= max_ctx) {
        pl->split_tokens = (int)((max_ctx + kTile - 1) / kTile * kTile);
        pl->max_splits = 1;
    } else {
        pl->split_tokens = T;
        pl->max_splits = (int)((max_ctx + T - 1) / T);
    }
    if (pl->max_splits > 65535 || sh->num_seqs > 65535) return PA_ERR_UNSUPPORTED;
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
    dim3 grid((Hkv * pl.n_chunks + kWaves - 1) / kWaves, pl.max_splits, S);
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
