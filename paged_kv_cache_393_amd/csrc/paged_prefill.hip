// paged_prefill.hip -- paged chunked-prefill attention for gfx950 (CDNA4)
// behind the C-ABI of include/paged_prefill.h.
//
// What is computed: every sequence's last n_q context tokens are queries; the
// query at position p attends causally to tokens 0 .. p through the block
// table (ybb.press page "LLM 推理 KV Cache 内存管理深度工程实践", section 7.3;
// t6page "KV cache" page, section "Chunked prefill：让 prefill 不阻塞 decode").
//
// Unlike decode, this is a dense contraction: a 512-token chunk of a
// Llama-3-8B layer does 4 d Hq flops per (query, context token) pair, far
// above the HBM ridge, so the work is laid out for the matrix cores
// (v_mfma_f32_16x16x32_bf16: A 16x32, B 32x16, lane l holding row / column l%16
// and k-elements 8*(l/16) .. +7; C lane l holding column l%16, rows 4*(l/16)+i).
//
// A "row" is a (query token, query head of the kv head's group) pair.  One
// workgroup takes 128 rows of one (sequence, kv head); each of its 4 waves
// owns 32 rows as two MFMA column blocks.  The workgroup streams the context
// in 32-token tiles through the block table: each thread loads 64 B of the
// next tile into registers (buffer loads whose range is each 16-token half's
// valid rows, so nothing past the context end is touched) while the current
// tile is computed from LDS, then stores them to the other LDS buffer (one
// barrier per tile; rows XOR-swizzled so the operand reads are conflict free):
//   * S^T = K Q^T per 16-token half: K rows (tokens) are the A operand, 16 B
//     per lane from LDS; the wave's query rows are the B operand, held in
//     registers for the whole context.
//   * causal mask and online softmax in the accumulator registers: lane l
//     holds column (row) l%16 and tokens 4*(l/16) + j of each half.
//   * O^T += V^T P^T: the 8 weights a lane holds ARE its B-operand k-elements,
//     under the token order e -> 16*(e/4) + 4*(l/16) + e%4; the A operand is
//     built from V with the same order: each lane loads, for those 8 tokens,
//     the contiguous dims chunk (l%16)*(D/16) .., and output block j takes
//     element j of each token's chunk (row m = dim m*(D/16) + j).  The weights
//     enter as a bf16 high part plus a bf16 remainder (two products), exact
//     to 2^-17 relative: a single bf16 rounding (2^-9) of the weights alone
//     exceeds a 2e-3 absolute bar on short contexts.
// Tokens past a column's position get weight 0; the accumulators leave lane l
// with row l%16 and the 4*(D/16) contiguous dims from 4*(D/16)*(l/16).

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "paged_prefill.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#ifndef PF_WAVES_PER_EU
#define PF_WAVES_PER_EU 2
#endif
// Column blocks per wave (2 fits two waves per SIMD; more registers per wave
// cost the occupancy that hides the loads' latency).
#ifndef PF_NC
#define PF_NC 2
#endif
#ifndef PF_XCD_MAP
#define PF_XCD_MAP 1
#endif

#ifndef PF_WAVES
#define PF_WAVES 8
#endif
constexpr int kWaves = PF_WAVES;           // waves per workgroup (rows share each staged tile)
constexpr int kThreads = 64 * kWaves;
constexpr int kNc = PF_NC;                 // MFMA column blocks (16 rows each) per wave
constexpr int kRowsPerWave = 16 * kNc;
constexpr int kRowsPerGroup = kRowsPerWave * kWaves;
constexpr int kTileTokens = 32;           // tokens per compute step (two 16-token MFMA halves)
#ifndef PF_LDS_TOKENS
#define PF_LDS_TOKENS 32
#endif
constexpr int kLdsTokens = PF_LDS_TOKENS;  // tokens per LDS-staged tile (compute steps of 32)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRsrcFlags = 0x00020000;     // word 3 of a raw buffer resource on CDNA3/CDNA4

struct PrefillParams {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *q_offsets;
    float *out;
    float scale_log2;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int max_blocks_per_seq;
    int log2_block_size;
    int num_seqs;
    int tiles_x;             // row tiles per (sequence, kv head)
};

// LDS staging of one kLdsTokens-token K/V tile of a kv head: row r (token t0 + r) is
// D*2 bytes = D/8 chunks of 16 B; chunk c of row r sits at position
// c ^ (r % (D/8)) so that the operand reads below (16 rows at one chunk, or
// one row at 16 chunks) touch distinct banks.
template <int D>
struct TileLds {
    static constexpr int kChunks = D / 8;
    static constexpr int kRowBytes = D * 2;
    static constexpr int kBytes = kLdsTokens * kRowBytes;            // one tensor
    static constexpr int kTotalChunks = kLdsTokens * kChunks;       // one tensor
    static constexpr int kChunksPerThread = (kTotalChunks + kThreads - 1) / kThreads;
    __device__ static int offset(int row, int chunk) {
        return row * kRowBytes + ((chunk ^ (row % kChunks)) * 16);
    }
};

template <int D>
__global__ __launch_bounds__(kThreads, PF_WAVES_PER_EU) void pa_prefill_kernel(const PrefillParams p) {
    constexpr int kSteps = D / 32;    // QK k-steps of 32 dims
    constexpr int kDpl = D / 16;      // V dims per lane = PV output blocks
    using TL = TileLds<D>;
    constexpr int kCpt = TL::kChunksPerThread;
    // [buffer][K, V] tiles, double-buffered: the next tile is loaded into
    // registers while the current one is computed from LDS.
    __shared__ __attribute__((aligned(16))) char lds_kv[2][2][TL::kBytes];
    __shared__ int lds_pmax[kWaves];

#if PF_XCD_MAP
    // Workgroup L runs on XCD L % 8 (round-robin dispatch).  (sequence, kv
    // head) pair P -- heaviest sequences first -- goes to XCD P % 8, and an
    // XCD runs its pairs in order, all row tiles of a pair together, so the
    // row tiles that read the same K/V share one L2.
    const int xcd = (int)(blockIdx.x % 8);
    const int y = (int)(blockIdx.x / 8);
    const int P = (y / p.tiles_x) * 8 + xcd;
    if (P >= p.num_kv_heads * p.num_seqs) return;    // uniform: the whole workgroup
    const int s = p.num_seqs - 1 - P / p.num_kv_heads;
    const int g = P % p.num_kv_heads;
    const int bx = p.tiles_x - 1 - y % p.tiles_x;
#else
    const int s = gridDim.z - 1 - blockIdx.z;
    const int bx = gridDim.x - 1 - blockIdx.x;
    const int g = blockIdx.y;
#endif
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int hgrp = lane >> 4;       // lane group: k-elements / accumulator rows
    const int l16 = lane & 15;
    const int G = p.group;
    const int q0 = p.q_offsets[s];
    const int nq = p.q_offsets[s + 1] - q0;
    const int R = nq * G;
    if (bx * kRowsPerGroup >= R) return;             // uniform: no row of the workgroup exists
    const int row0 = bx * kRowsPerGroup + wave * kRowsPerWave;
    const bool wave_live = row0 < R;
    const int ctx = p.context_lens[s];
    const int Hq = p.num_q_heads;
    const int Hkv = p.num_kv_heads;
    const uint32_t rb32 = (uint32_t)(Hkv * D * 2);     // bytes of one token slot (all kv heads)
    const char *kbase = (const char *)p.k + (int64_t)g * D * 2;
    const char *vbase = (const char *)p.v + (int64_t)g * D * 2;
    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const int bs_log2 = p.log2_block_size;
    const int bs_mask = (1 << bs_log2) - 1;

    // Columns of this lane: row r = row0 + 16 cb + l16 -> query token r / G,
    // head g*G + r % G, position ctx - nq + r / G.  Columns past R compute
    // with position 0 and are not stored.
    int pos[kNc];
    bool colv[kNc];
    bf16x8_t qop[kNc][kSteps];
#pragma unroll
    for (int cb = 0; cb < kNc; ++cb) {
        const int r = row0 + 16 * cb + l16;
        colv[cb] = r < R;
        const int i = colv[cb] ? r / G : 0;
        const int hh = colv[cb] ? r - i * G : 0;
        pos[cb] = colv[cb] ? ctx - nq + i : 0;
        const uint16_t *qrow = p.q + ((int64_t)(q0 + i) * Hq + g * G + hh) * D;
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            u32x4_t w = *(const u32x4_t *)(qrow + 32 * st + 8 * hgrp);
            if (!colv[cb]) w = u32x4_t{0u, 0u, 0u, 0u};
            qop[cb][st] = __builtin_bit_cast(bf16x8_t, w);
        }
    }
    int pmax = pos[0], pmin = pos[0];
#pragma unroll
    for (int cb = 1; cb < kNc; ++cb) {
        pmax = max(pmax, pos[cb]);
        pmin = min(pmin, pos[cb]);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        pmax = max(pmax, __shfl_xor(pmax, off));
        pmin = min(pmin, __shfl_xor(pmin, off));
    }
    if (lane == 0) lds_pmax[wave] = wave_live ? pmax : -1;
    __syncthreads();
    int wg_pmax = lds_pmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) wg_pmax = max(wg_pmax, lds_pmax[w]);
    const int n_tiles = wg_pmax / kLdsTokens + 1;      // the workgroup's LDS tiles (uniform)
    const int my_steps = pmax / kTileTokens + 1;       // this wave's compute steps

    // This thread's share of a tile's loads: flat chunks threadIdx.x + j * kThreads
    // (row = flat / chunks per row, chunk = flat % chunks per row).
    const int ld_chunk = (int)threadIdx.x % TL::kChunks;
    u32x4_t pre_k[kCpt], pre_v[kCpt];
    auto ld_ok = [&](int j) __attribute__((always_inline)) {
        return TL::kTotalChunks % kThreads == 0 || (int)threadIdx.x + j * kThreads < TL::kTotalChunks;
    };
    auto ld_row = [&](int j) __attribute__((always_inline)) {
        return ((int)threadIdx.x + j * kThreads) / TL::kChunks;
    };
    auto load_tile = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kCpt; ++j) {
            if (!ld_ok(j)) continue;
            const int row = ld_row(j);                                // 0 .. kLdsTokens-1
            const int tb = t0 + (row & ~15);                          // the row's 16-token half
            const int rows = min(16, max(0, ctx - tb));
            const int phys = rows > 0 ? table[tb >> bs_log2] : 0;
            const int64_t slot0 = ((int64_t)phys << bs_log2) + (tb & bs_mask);
            const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(kbase + slot0 * rb32), 0, rows * (int)rb32, kRsrcFlags);
            const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(vbase + slot0 * rb32), 0, rows * (int)rb32, kRsrcFlags);
            const int off = (int)((uint32_t)(row & 15) * rb32 + (uint32_t)(ld_chunk * 16));
            pre_k[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
            pre_v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kCpt; ++j) {
            if (!ld_ok(j)) continue;
            const int row = ld_row(j);
            const int o = TL::offset(row, ld_chunk);
            *(u32x4_t *)(&lds_kv[buf][0][o]) = pre_k[j];
            *(u32x4_t *)(&lds_kv[buf][1][o]) = pre_v[j];
        }
    };

    f32x4_t acc[kDpl][kNc];
#pragma unroll
    for (int j = 0; j < kDpl; ++j)
#pragma unroll
        for (int cb = 0; cb < kNc; ++cb) acc[j][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[kNc], l_run[kNc];
#pragma unroll
    for (int cb = 0; cb < kNc; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.f;
    }

    load_tile(0);
    store_tile(0);
    for (int tile = 0; tile < n_tiles; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < n_tiles) load_tile((tile + 1) * kLdsTokens);   // in flight during the compute
        __syncthreads();      // tile `tile` is in LDS; every wave is done with the other buffer
#pragma unroll 1
        for (int sub = 0; sub < kLdsTokens / kTileTokens; ++sub) {
          const int step = tile * (kLdsTokens / kTileTokens) + sub;
          const int t0 = step * kTileTokens;
          if (wave_live && step < my_steps) {
            const char *kl = lds_kv[buf][0] + sub * kTileTokens * TL::kRowBytes;
            const char *vl = lds_kv[buf][1] + sub * kTileTokens * TL::kRowBytes;
            // ---- S^T = K Q^T from LDS, masked online softmax, weights as B operand
            bf16x8_t pop[kNc], pop_lo[kNc];
            float alpha[kNc];
            f32x4_t sacc[2][kNc];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                bf16x8_t kop[kSteps];
#pragma unroll
                for (int st = 0; st < kSteps; ++st)
                    kop[st] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(kl + TL::offset(16 * bb + l16, 4 * st + hgrp)));
#pragma unroll
                for (int cb = 0; cb < kNc; ++cb) {
                    sacc[bb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < kSteps; ++st)
                        sacc[bb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[st], qop[cb][st], sacc[bb][cb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                float sc[8];
                float mx = -INFINITY;
                if (t0 + kTileTokens - 1 <= pmin) {   // every token of the tile is visible
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sc[e] = sacc[e >> 2][cb][e & 3] * p.scale_log2;
                        mx = fmaxf(mx, sc[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int t = t0 + 16 * (e >> 2) + 4 * hgrp + (e & 3);
                        sc[e] = t <= pos[cb] ? sacc[e >> 2][cb][e & 3] * p.scale_log2 : -INFINITY;
                        mx = fmaxf(mx, sc[e]);
                    }
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run[cb], mx);   // finite: token 0 <= every position
                alpha[cb] = __builtin_amdgcn_exp2f(m_run[cb] - m_new);
                float pr[8], psum = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pr[e] = __builtin_amdgcn_exp2f(sc[e] - m_new);
                    psum += pr[e];
                }
                l_run[cb] = l_run[cb] * alpha[cb] + psum;
                m_run[cb] = m_new;
                // the weights as a bf16 high part plus a bf16 remainder, both
                // rounded to nearest even: hi + lo is the fp32 weight to 2^-17
                u32x4_t pw, pl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x2_t w2 = f32x2_t{pr[2 * e], pr[2 * e + 1]};
                    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(w2, bf16x2_t));
                    const f32x2_t r2 = w2 - f32x2_t{__uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
                    pw[e] = hi;
                    pl[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2_t));
                }
                pop[cb] = __builtin_bit_cast(bf16x8_t, pw);
                pop_lo[cb] = __builtin_bit_cast(bf16x8_t, pl);
            }
            bool moved = false;
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) moved = moved || alpha[cb] != 1.f;
            if (__ballot(moved)) {
#pragma unroll
                for (int j = 0; j < kDpl; ++j)
#pragma unroll
                    for (int cb = 0; cb < kNc; ++cb) acc[j][cb] *= alpha[cb];
            }
            // ---- O^T += V^T P^T: the lane's dims of its 8 tokens (row order
            // e -> 16 (e/4) + 4 hgrp + e%4), output block j from element j.
            uint32_t vw[8][kDpl / 2];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = 16 * (e >> 2) + 4 * hgrp + (e & 3);
                if constexpr (D == 128) {
                    const u32x4_t c = *(const u32x4_t *)(vl + TL::offset(row, l16));
                    vw[e][0] = c.x; vw[e][1] = c.y; vw[e][2] = c.z; vw[e][3] = c.w;
                } else {
                    const u32x2_t c = *(const u32x2_t *)(vl + TL::offset(row, l16 >> 1) + 8 * (l16 & 1));
                    vw[e][0] = c.x; vw[e][1] = c.y;
                }
            }
#pragma unroll
            for (int j = 0; j < kDpl; ++j) {
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t a;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a[e] = __builtin_amdgcn_perm(vw[2 * e + 1][j >> 1], vw[2 * e][j >> 1], sel);
                const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
                for (int cb = 0; cb < kNc; ++cb) {
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[cb], acc[j][cb], 0, 0, 0);
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo[cb], acc[j][cb], 0, 0, 0);
                }
            }
          }
        }
        // The next tile goes to the other buffer, which every wave finished
        // reading before the barrier above.
        if (tile + 1 < n_tiles) store_tile(buf ^ 1);
    }

    if (!wave_live) return;
    // ---- the four lane groups hold partial sums over different tokens
#pragma unroll
    for (int cb = 0; cb < kNc; ++cb) {
        float l = l_run[cb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (!colv[cb]) continue;
        const int r = row0 + 16 * cb + l16;
        const int i = r / G;
        const int hh = r - i * G;
        const float inv = 1.f / l;
        float *dst = p.out + ((int64_t)(q0 + i) * Hq + g * G + hh) * D + 4 * kDpl * hgrp;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < kDpl; j += 4)
                *(f32x4_t *)(dst + e * kDpl + j) = f32x4_t{acc[j][cb][e] * inv, acc[j + 1][cb][e] * inv,
                                                           acc[j + 2][cb][e] * inv, acc[j + 3][cb][e] * inv};
    }
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}
bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

}  // namespace

extern "C" int paged_attn_prefill(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *q_offsets, float scale, float *out,
                                  const pa_prefill_shape *sh, void *stream) {
    if (!sh) return PA_ERR_NULL;
    if (sh->num_seqs < 0 || sh->num_q_heads < 1 || sh->num_kv_heads < 1 ||
        sh->max_blocks_per_seq < 1 || sh->num_blocks < 1 || sh->max_q_len < 1)
        return PA_ERR_SHAPE;
    if (sh->num_q_heads % sh->num_kv_heads) return PA_ERR_SHAPE;
    if (sh->head_dim != 64 && sh->head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(sh->block_size) || sh->block_size < 16 || sh->block_size > 4096)
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)sh->max_blocks_per_seq * sh->block_size >= ((int64_t)1 << 30)) return PA_ERR_UNSUPPORTED;
    const int group = sh->num_q_heads / sh->num_kv_heads;
    const int64_t rows = (int64_t)sh->max_q_len * group;
    const int64_t tiles = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
    if (rows >= ((int64_t)1 << 30) || tiles > 0x7fffffff || sh->num_kv_heads > 65535 ||
        sh->num_seqs > 65535)
        return PA_ERR_UNSUPPORTED;
    if (sh->num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !q_offsets || !out)
        return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return PA_ERR_ALIGNMENT;
    PrefillParams p;
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k_cache;
    p.v = (const uint16_t *)v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.q_offsets = q_offsets;
    p.out = out;
    p.scale_log2 = scale * kLog2e;
    p.num_q_heads = sh->num_q_heads;
    p.num_kv_heads = sh->num_kv_heads;
    p.group = group;
    p.max_blocks_per_seq = sh->max_blocks_per_seq;
    p.log2_block_size = ilog2(sh->block_size);
    p.num_seqs = sh->num_seqs;
    p.tiles_x = (int)tiles;
#if PF_XCD_MAP
    const int64_t pairs = (int64_t)sh->num_kv_heads * sh->num_seqs;
    const int64_t n_wg = 8 * ((pairs + 7) / 8) * tiles;
    if (n_wg >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)n_wg);
#else
    const dim3 grid((unsigned)tiles, (unsigned)sh->num_kv_heads, (unsigned)sh->num_seqs);
#endif
    const dim3 block(kThreads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (sh->head_dim == 128) hipLaunchKernelGGL(pa_prefill_kernel<128>, grid, block, 0, st, p);
    else hipLaunchKernelGGL(pa_prefill_kernel<64>, grid, block, 0, st, p);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
