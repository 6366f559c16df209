// paged_attn.hip -- PagedAttention decode for gfx950 (CDNA4) behind the C-ABI
// of include/paged_attn.h.
//
// What is computed: for each sequence s and query head h, the decode query
// attends over the sequence's context gathered through its block table, with
// G = Hq / Hkv consecutive query heads sharing kv head h / G, scores
// scale * q.k and one exact softmax over the whole context (ybb.press page
// "LLM 推理 KV Cache 内存管理深度工程实践", sections 2.2 and 6.2; t6page
// "KV cache" page, section "PagedAttention 的算子").  The int8 variant
// dequantizes code * per-(slot, kv head) scale, the fp8 variant reads the
// cache cast to FP8 E4M3 (both: same ybb.press page, 6.1).
//
// Work decomposition.  A "unit" is (kv head, chunk of <= 16 query heads of
// its group); one wave serves one unit.  A workgroup holds four waves for four
// consecutive units (a "unit group"), which read the same tokens: the kv
// heads' rows of a token slot are adjacent in memory.  The context of every
// sequence is cut into 16-token tiles, and the tiles of all sequences are laid
// end to end (sequence-major) into one work list, the same for every unit
// group.  The grid is persistent -- as many workgroups as the GPU holds at
// once -- and each workgroup takes an equal share ("item") of the list, so
// every compute unit streams about the same number of bytes whatever the mix
// of context lengths.  An item may hold the tail of one sequence, whole
// sequences and the head of another; each such piece is a run of tiles with a
// private online-softmax state.  A piece that covers a whole sequence writes
// the output directly.  Otherwise it stores an unnormalised partial (acc, max,
// sum), and a second kernel merges the partials of each split sequence with
// log-sum-exp weights, in a fixed order, so results are reproducible.  (The
// kernel boundary is what makes the partials of all workgroups visible: the
// L2 caches of the eight XCDs are not coherent with each other, and making
// them so inside the kernel costs a full L2 write-back per partial.)
//
// Per 16-token tile and wave, on the matrix cores (v_mfma_f32_16x16x16_bf16):
//   * S = K Q^T: K rows (tokens) are the A operand, loaded 16 B per lane
//     (token l%16; the four lane groups take complementary dims); the unit's
//     query heads (zero-padded to 16) are the B operand, loaded once per piece.
//     Lane l gets the scores of head l%16 for tokens 4*(l/16)..+3.
//   * online softmax in those registers: tile max over the 16 tokens (two
//     xor-shuffles), running max, rescale factor, p = 2^(s*scale*log2e - m).
//   * O^T += V^T P^T: the probabilities already sit in the B operand layout
//     (token rows 4*(l/16).., head column l%16).  They are split into a bf16
//     high part and a bf16 remainder (v_cvt_pk_bf16_f32, round to nearest
//     even), two MFMAs per output block, which keeps the weights exact to
//     2^-17 relative.  V is the A operand: lane l
//     loads dims (l%16)*(D/16) .. +D/16-1 of tokens 4*(l/16)+i, so one load
//     instruction reads four whole token rows, and a byte permute turns them
//     into the operand of each output block (block j, row m = dim m*(D/16)+j).
//     The fp32 accumulator then holds, in lane l, head l%16 and the
//     4*(D/16) dims starting at 4*(D/16)*(l/16).
//   * the loads of the next tiles are in flight while a tile is processed
//     (register pipeline).
// Rows of the last tile past the context end are slots of the same allocated
// block; the loads do not touch them (buffer range) and they are selected away
// (score -inf, V and int8 V scale replaced by 0), so padding cannot reach the
// output.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "paged_attn.h"

namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Tuning knobs (compile-time): tiles in flight per wave, and the minimum
// number of waves per SIMD the register allocation must allow.
#ifndef PA_STAGES
#define PA_STAGES 2
#endif
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 2
#endif

constexpr int kTile = 16;           // tokens per tile (MFMA rows of S, k of PV)
constexpr int kWaves = 4;           // waves (units) per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kHeads = 16;          // query heads per unit (MFMA columns)
constexpr int kWindow = 128;        // block ids held in registers (two per lane)
constexpr int kMinItemTiles = 4;    // shortest balanced item
constexpr int kMaxItems = 4096;     // balanced items per unit group (>= workgroups launched)
constexpr int kLdsSeqs = 2048;      // sequences whose tile prefix and length are kept in LDS
constexpr float kLog2e = 1.4426950408889634f;
// Element kinds of the KV cache.
enum KvKind : int { kBf16 = 0, kInt8 = 1, kFp8 = 2 };
// Word 3 of a raw (unformatted, stride 0) buffer resource on CDNA3/CDNA4.
constexpr int kRsrcFlags = 0x00020000;
// Cache-policy operand of the V buffer loads: the non-temporal bit (nt).
// Every V byte is read once per call, and a V load instruction reads whole
// 256-B runs, so the streamed lines are not kept in the caches; with it the
// Llama-3-8B batch step went from 112 to 102 us, the 70B-shaped layers from
// 1344 to 1210 us.  K loads keep the default policy: a K load instruction
// reads 64 B (32 B for 1-byte caches) of each of 16 token rows and the rest of
// each 128-B line comes with the next instructions, which then hit in the
// cache (int8 215 -> 202 us, fp8 198 -> 193 us against nt on K too).  The
// int8 scale loads keep it as well: a scale line holds the scales of all kv
// heads of 4 slots and is read by both workgroups of a slot.
constexpr int kStreamPolicy = 2;

struct Params {
    const uint16_t *q;       // bf16 [S, Hq, D]
    const void *k;           // [NB, bs, Hkv, D] bf16, int8 or fp8 (E4M3)
    const void *v;
    const float *k_scales;   // [NB, bs, Hkv] (int8 only)
    const float *v_scales;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *out;              // fp32 [S, Hq, D]
    float *part;             // partial records (workspace)
    int32_t *seg_items;      // [S, 2] first and last item holding each sequence (workspace)
    float scale_log2;        // softmax scale * log2(e)
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;               // Hq / Hkv
    int n_chunks;            // ceil(group / kHeads)
    int units;               // Hkv * n_chunks
    int rec_heads;           // min(group, kHeads): heads per partial record
    int max_blocks_per_seq;
    int max_ctx;             // max_blocks_per_seq * block_size
    int log2_block_size;
    int item_tiles;          // > 0: fixed item length in tiles; 0: balanced
    int max_pieces;          // partial records per (unit group, wave)
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Signed byte b of w as float (exact).
__device__ __forceinline__ float i8_at(uint32_t w, int b) {
    return (float)(int)(int8_t)((w >> (8 * b)) & 0xffu);
}

// Bits of the bf16 pair (x, y), x in the low half, from two floats whose low
// 16 bits are zero or are to be dropped.
__device__ __forceinline__ uint32_t pack_hi16(float x, float y) {
    return __builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
}

// Four signed bytes -> four bf16 (exact: |code| <= 128 has at most 8 significant bits).
__device__ __forceinline__ bf16x4_t i8x4_to_bf16x4(uint32_t w) {
    return __builtin_bit_cast(bf16x4_t, u32x2_t{pack_hi16(i8_at(w, 0), i8_at(w, 1)),
                                                pack_hi16(i8_at(w, 2), i8_at(w, 3))});
}

// Two FP8 E4M3 codes (bytes 2*hi, 2*hi + 1 of w) -> their bf16 pair, low half
// first.  Exact: every E4M3 value (subnormals and NaN included) is a bf16
// value, and the scale operand is 1.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// Four FP8 E4M3 codes -> four bf16 (exact).
__device__ __forceinline__ bf16x4_t fp8x4_to_bf16x4(uint32_t w) {
    return __builtin_bit_cast(bf16x4_t, u32x2_t{fp8x2_to_bf16x2<false>(w), fp8x2_to_bf16x2<true>(w)});
}

// Order this wave's LDS writes before its following LDS reads (other lanes'
// data); LDS requests of one wave complete in order.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (compile-time unrolled).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Tiles of a sequence in the work list; an empty context still takes one
// (empty) tile, so that its output row is written.
__device__ __forceinline__ int tiles_of(int ctx) { return ctx > 0 ? (ctx + kTile - 1) / kTile : 1; }

// Items of the work list: either fixed-length (`fixed` tiles each) or an even
// split of the T tiles into n items; item j covers tiles [lo(j), lo(j + 1)).
struct Items {
    int T;
    int n;
    int fixed;
    __device__ __forceinline__ int lo(int j) const {
        if (fixed) return (int)min((int64_t)j * fixed, (int64_t)T);
        return (int)((int64_t)j * T / n);
    }
    // Index of the item holding tile x (0 <= x < T).  For the even split every
    // item is non-empty (n <= T), so the estimate is off by at most one.
    __device__ __forceinline__ int of(int x) const {
        if (fixed) return x / fixed;
        int c = (int)((int64_t)x * n / T);
        if (c + 1 < n && lo(c + 1) <= x) ++c;
        return c;
    }
};

template <int D, int KV>
struct Layout {
    static constexpr int kElem = KV == kBf16 ? 2 : 1;          // bytes per cache element
    static constexpr int kKElemsPerLoad = 16 / kElem;          // K dims per 16-B load
    static constexpr int kKLoads = D / (4 * kKElemsPerLoad);   // 16-B K loads per lane per tile
    static constexpr int kSteps = D / 16;                      // QK MFMA k-steps (4 dims x 4 groups)
    static constexpr int kStepsPerLoad = kKElemsPerLoad / 4;
    static constexpr int kDpl = D / 16;                        // V dims per lane and token = PV blocks
    static constexpr int kVBytes = kDpl * kElem;               // 16, 8 or 4
    using VReg = typename std::conditional<
        kVBytes == 16, u32x4_t, typename std::conditional<kVBytes == 8, u32x2_t, uint32_t>::type>::type;
    // First dim of QK step `st` for lane group `lg`; the step covers 4 dims.
    __device__ static constexpr int step_dim(int st, int lg) {
        return (st / kStepsPerLoad) * 4 * kKElemsPerLoad + kKElemsPerLoad * lg +
               4 * (st % kStepsPerLoad);
    }
};

template <int D, int KV>
struct TileRegs {
    using L = Layout<D, KV>;
    u32x4_t k[L::kKLoads];
    typename L::VReg v[4];   // token rows 4*(l/16) + i
    float ks;                // int8: K scale of token row l%16
    float vs;                // int8: V scale of token row l%16
};

// 32-bit word w of a V register.
template <typename VR>
__device__ __forceinline__ uint32_t vword(const VR &r, int w) {
    if constexpr (std::is_same<VR, uint32_t>::value) return r;
    else return r[w];
}

// A operand of PV block j: element j of the four token rows, as bf16x4.
template <int D, int KV>
__device__ __forceinline__ bf16x4_t v_operand(const typename Layout<D, KV>::VReg (&v)[4], int j) {
    u32x2_t r;
    if constexpr (KV == kInt8) {
        const int w = j >> 2, b = j & 3;
        r.x = pack_hi16(i8_at(vword(v[0], w), b), i8_at(vword(v[1], w), b));
        r.y = pack_hi16(i8_at(vword(v[2], w), b), i8_at(vword(v[3], w), b));
    } else if constexpr (KV == kFp8) {
        // Byte b of rows (0, 1) and of rows (2, 3) side by side, then converted.
        const int w = j >> 2, b = j & 3;
        const uint32_t sel = (uint32_t)b | ((uint32_t)(4 + b) << 8) | 0x0c0c0000u;
        r.x = fp8x2_to_bf16x2<false>(__builtin_amdgcn_perm(vword(v[1], w), vword(v[0], w), sel));
        r.y = fp8x2_to_bf16x2<false>(__builtin_amdgcn_perm(vword(v[3], w), vword(v[2], w), sel));
    } else {
        const int w = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        r.x = __builtin_amdgcn_perm(vword(v[1], w), vword(v[0], w), sel);
        r.y = __builtin_amdgcn_perm(vword(v[3], w), vword(v[2], w), sel);
    }
    return __builtin_bit_cast(bf16x4_t, r);
}

template <int D, int KV>
__global__ __launch_bounds__(kThreads, PA_WAVES_PER_EU) void pa_decode_kernel(const Params p) {
    constexpr bool INT8 = KV == kInt8;
    using L = Layout<D, KV>;
    constexpr int kDpl = L::kDpl;
    static_assert(L::kKLoads >= 1, "head_dim");

    __shared__ int lds_incl[kLdsSeqs];   // inclusive prefix of tiles per sequence
    __shared__ int lds_ctx[kLdsSeqs];    // context length per sequence
    __shared__ int lds_red[kWaves];
    __shared__ int lds_found[2];
    __shared__ __attribute__((aligned(16))) float lds_sc[kWaves][2 * kTile];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4;      // lane group: score rows / PV k rows
    const int l16 = lane & 15;     // K token row, head column
    const int S = p.num_seqs;
    const int ug = blockIdx.y;                    // unit group
    const int unit = ug * kWaves + wave;          // this wave's unit
    const bool active = unit < p.units;
    // Context length as used here: clamped to what the table row can address.
    auto ctx_of = [&](int s) __attribute__((always_inline)) {
        return min(max(p.context_lens[s], 0), p.max_ctx);
    };

    // ---- Tiles per sequence: the list length T (the host checked that it
    // fits in int) and, for batches of up to kLdsSeqs, the inclusive prefix
    // and the context lengths in LDS. ----
    const bool in_lds = S <= kLdsSeqs;
    int T = 0;
    for (int c0 = 0; c0 < S; c0 += kThreads) {
        const int s = c0 + threadIdx.x;
        const int ctx = s < S ? ctx_of(s) : 0;
        const int n = s < S ? tiles_of(ctx) : 0;
        int incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        if (lane == 63) lds_red[wave] = incl;
        __syncthreads();
        int before = T, chunk_total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            before += w < wave ? lds_red[w] : 0;
            chunk_total += lds_red[w];
        }
        if (in_lds && s < S) {
            lds_incl[s] = incl + before;
            lds_ctx[s] = ctx;
        }
        __syncthreads();
        T += chunk_total;
    }
    Items items;
    items.T = T;
    items.fixed = p.item_tiles;
    items.n = p.item_tiles ? (items.T + p.item_tiles - 1) / p.item_tiles
                           : min((int)gridDim.x, (items.T + kMinItemTiles - 1) / kMinItemTiles);

    // Unit constants.
    const int g = active ? unit / p.n_chunks : 0;
    const int chunk = active ? unit - g * p.n_chunks : 0;
    const int h_base = g * p.group + chunk * kHeads;
    const int n_heads = min(kHeads, p.group - chunk * kHeads);
    const int Hq = p.num_q_heads;
    const int Hkv = p.num_kv_heads;
    const int bs_log2 = p.log2_block_size;
    const int bs_mask = (1 << bs_log2) - 1;
    const int64_t row_bytes = (int64_t)Hkv * D * L::kElem;   // one token slot, all kv heads
    const uint32_t rb32 = (uint32_t)row_bytes;
    const char *kbase = (const char *)p.k + (int64_t)g * D * L::kElem;
    const char *vbase = (const char *)p.v + (int64_t)g * D * L::kElem;
    const size_t rec_floats = (size_t)p.rec_heads * (D + 2);
    float *rec_base = p.part + ((size_t)ug * p.max_pieces * kWaves + wave) * rec_floats;
    const size_t rec_stride = (size_t)kWaves * rec_floats;   // between pieces
    const bool live = l16 < n_heads;                          // lane's head column is real
    const int dim0 = lg * 4 * kDpl;   // first of this lane's 4*kDpl output dims

    // Per-lane byte offsets of a tile's loads, fixed for the whole kernel.
    const int k_off = (int)((uint32_t)l16 * rb32 + (uint32_t)(L::step_dim(0, lg) * L::kElem));
    int v_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v_off[i] = (int)((uint32_t)(4 * lg + i) * rb32 + (uint32_t)(l16 * L::kVBytes));
    const int s_off = (int)(((uint32_t)l16 * (uint32_t)Hkv + (uint32_t)g) * 4u);

    // Per-piece operands: the query heads (B operand of S = K Q^T; zero for
    // padding heads) and the block ids of the piece as a register window of
    // kWindow entries (lane i holds ids first + i and first + 64 + i).
    struct Meta {
        bf16x4_t q[L::kSteps];
        int w0, w1, first;
    };
    auto load_window = [&](Meta &m, const int32_t *table, int blk_first, int blk_end)
        __attribute__((always_inline)) {
        m.first = blk_first;
        m.w0 = (blk_first + lane < blk_end) ? table[blk_first + lane] : 0;
        m.w1 = (blk_first + 64 + lane < blk_end) ? table[blk_first + 64 + lane] : 0;
    };
    // Meta of the piece of sequence s holding tokens [t_begin, t_end).
    auto load_meta = [&](Meta &m, int s, int t_begin, int t_end) __attribute__((always_inline)) {
        const uint16_t *qrow = p.q + ((int64_t)s * Hq + h_base + (live ? l16 : 0)) * D;
#pragma unroll
        for (int st = 0; st < L::kSteps; ++st) {
            u32x2_t w = *(const u32x2_t *)(qrow + L::step_dim(st, lg));
            if (!live) w = u32x2_t{0u, 0u};
            m.q[st] = __builtin_bit_cast(bf16x4_t, w);
        }
        load_window(m, p.block_tables + (int64_t)s * p.max_blocks_per_seq, t_begin >> bs_log2,
                    ((t_end - 1) >> bs_log2) + 1);
    };

    // Tile buffers of the register pipeline, kept across the pieces of an
    // item: a piece whose tile count is a multiple of the depth loads the next
    // piece's first tile into buf[0] in its last step, in place of a re-load
    // past its end, and `pre_ok` tells the next piece that it is there.
    constexpr int kStages = PA_STAGES;
    static_assert(kStages >= 2 && kStages <= 6, "pipeline depth");
    TileRegs<D, KV> buf[kStages];
    bool pre_ok = false;

    // One piece: tiles [ta, tb) of sequence s for this wave's unit, with its
    // operands in `mt`.  Items `first` .. `last` are those that hold the
    // sequence; `item` holds this piece.  The item's next piece (if
    // next_rows > 0) is sequence s + 1 from token 0, with operands `mnx`;
    // next_rows is the number of valid rows of its first tile.
    auto process = [&](int s, int ctx, int ta, int tb, int first, int last, int item, Meta &mt,
                       Meta &mnx, int next_rows) __attribute__((always_inline)) {
        const int64_t row0 = (int64_t)s * Hq + h_base;   // output row of head column 0
        if (ctx == 0) {   // empty context: the output row is zero (always one whole piece)
            if (live) {
                float *dst = p.out + (row0 + l16) * D + dim0;
#pragma unroll
                for (int e = 0; e < 4 * kDpl; e += 4) *(f32x4_t *)(dst + e) = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            pre_ok = false;
            return;
        }
        const int t_begin = ta * kTile;
        const int t_end = min(ctx, tb * kTile);
        const int n_tiles = tb - ta;
        const bf16x4_t(&qop)[L::kSteps] = mt.q;

        // The window is refilled when a tile leaves it, so the tile loop makes
        // no dependent memory access unless a piece spans more than kWindow
        // blocks.
        const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
        const int blk_end = ((t_end - 1) >> bs_log2) + 1;
        // Token-slot index phys * block_size + slot of the first token of tile `tile` (uniform).
        auto tile_slot = [&](int tile) __attribute__((always_inline)) -> int64_t {
            const int t0 = t_begin + tile * kTile;
            const int blk = t0 >> bs_log2;
            if (blk - mt.first >= kWindow) load_window(mt, table, blk, blk_end);
            const int idx = blk - mt.first;
            const int phys = idx < 64 ? __builtin_amdgcn_readlane(mt.w0, idx)
                                      : __builtin_amdgcn_readlane(mt.w1, idx - 64);
            return ((int64_t)phys << bs_log2) + (t0 & bs_mask);
        };

        // Tile loads are raw buffer loads: a uniform buffer resource per tile
        // whose range is the tile's valid rows, plus the fixed per-lane offsets.
        // A tile never crosses a block (block_size is a multiple of 16); rows
        // at or past the context end fall outside the range and read as 0
        // without touching memory.
        auto load_rows = [&](TileRegs<D, KV> &r, int64_t slot0, int rows) __attribute__((always_inline)) {
            const int range = rows * (int)rb32;
            const __amdgpu_buffer_rsrc_t kr =
                __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + slot0 * row_bytes), 0, range, kRsrcFlags);
            const __amdgpu_buffer_rsrc_t vr =
                __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + slot0 * row_bytes), 0, range, kRsrcFlags);
#pragma unroll
            for (int m = 0; m < L::kKLoads; ++m)
                r.k[m] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                             kr, k_off + m * 4 * L::kKElemsPerLoad * L::kElem, 0, 0));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (L::kVBytes == 16)
                    r.v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vr, v_off[i], 0, kStreamPolicy));
                else if constexpr (L::kVBytes == 8)
                    r.v[i] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(vr, v_off[i], 0, kStreamPolicy));
                else
                    r.v[i] = __builtin_amdgcn_raw_buffer_load_b32(vr, v_off[i], 0, kStreamPolicy);
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
        auto load_tile = [&](TileRegs<D, KV> &r, int tile) __attribute__((always_inline)) {
            load_rows(r, tile_slot(tile), min(kTile, t_end - (t_begin + tile * kTile)));
        };
        // Tile k of the pipeline: this piece's tile k; past the end, the next
        // piece's first tile if there is one (its first block is lane 0 of
        // its window), else this piece's last tile again (a cache hit).  The
        // branches are uniform and every path issues the same loads into r.
        auto load_ext = [&](TileRegs<D, KV> &r, int k) __attribute__((always_inline)) {
            int64_t slot0;
            int rows;
            if (k < n_tiles) {
                slot0 = tile_slot(k);
                rows = min(kTile, t_end - (t_begin + k * kTile));
            } else if (next_rows > 0) {
                slot0 = (int64_t)__builtin_amdgcn_readlane(mnx.w0, 0) << bs_log2;
                rows = next_rows;
            } else {
                slot0 = tile_slot(n_tiles - 1);
                rows = min(kTile, t_end - (t_begin + (n_tiles - 1) * kTile));
            }
            load_rows(r, slot0, rows);
        };

        // Online-softmax state of head l16 (the same in the four lane groups)
        // and the PV accumulator: block j, element i = dim kDpl*(4*lg+i)+j.
        float m_run = -INFINITY;
        float l_run = 0.f;   // this lane's share (its four token rows)
        f32x4_t acc[kDpl];
#pragma unroll
        for (int j = 0; j < kDpl; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto compute_tile = [&](TileRegs<D, KV> &r, int tile) __attribute__((always_inline)) {
            const int t0 = t_begin + tile * kTile;
            if constexpr (INT8) {
                wave_lds_sync();
                if (lane < kTile) lds_sc[wave][lane] = r.ks;
                else if (lane < 2 * kTile) lds_sc[wave][lane] = r.vs;
            }
            // S = K Q^T: rows = tokens, columns = heads.
            f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < L::kSteps; ++st) {
                const int m = st / L::kStepsPerLoad;
                const int sub = st % L::kStepsPerLoad;
                bf16x4_t a;
                if constexpr (KV == kInt8) {
                    a = i8x4_to_bf16x4(r.k[m][sub]);
                } else if constexpr (KV == kFp8) {
                    a = fp8x4_to_bf16x4(r.k[m][sub]);
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
            bool valid[4];
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                valid[i] = t0 + 4 * lg + i < t_end;
                const float x = sacc[i] * (INT8 ? p.scale_log2 * ks[i] : p.scale_log2);
                sc[i] = valid[i] ? x : -INFINITY;
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
                pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);   // 0 for masked rows
                psum += pr[i];
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            if (__ballot(alpha != 1.f)) {   // the running max moved for some head
#pragma unroll
                for (int j = 0; j < kDpl; ++j) acc[j] *= alpha;
            }
            // B operand of PV: the weights (times the int8 V scale) as a bf16
            // high part plus a bf16 remainder, both rounded to nearest even:
            // hi + lo equals the fp32 weight to within 2^-17 relative.
            f32x2_t w01, w23;
            if constexpr (INT8) {
                w01 = f32x2_t{valid[0] ? pr[0] * vsc[0] : 0.f, valid[1] ? pr[1] * vsc[1] : 0.f};
                w23 = f32x2_t{valid[2] ? pr[2] * vsc[2] : 0.f, valid[3] ? pr[3] * vsc[3] : 0.f};
            } else {
                w01 = f32x2_t{pr[0], pr[1]};
                w23 = f32x2_t{pr[2], pr[3]};
            }
            const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(w01, bf16x2_t));
            const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(w23, bf16x2_t));
            const f32x2_t r01 = w01 - f32x2_t{bf16_lo(h01), bf16_hi(h01)};
            const f32x2_t r23 = w23 - f32x2_t{bf16_lo(h23), bf16_hi(h23)};
            const bf16x4_t bhi = __builtin_bit_cast(bf16x4_t, u32x2_t{h01, h23});
            const bf16x4_t blo = __builtin_bit_cast(
                bf16x4_t, u32x2_t{__builtin_bit_cast(uint32_t, __builtin_convertvector(r01, bf16x2_t)),
                                  __builtin_bit_cast(uint32_t, __builtin_convertvector(r23, bf16x2_t))});
            // Rows past the context end (last tile only) are replaced by zeros.
            if (t_end - t0 < kTile) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!valid[i]) r.v[i] = typename L::VReg{};
            }
#pragma unroll
            for (int j = 0; j < kDpl; ++j) {
                const bf16x4_t a = v_operand<D, KV>(r.v, j);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bhi, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, blo, acc[j], 0, 0, 0);
            }
        };

        // Register pipeline of kStages tile buffers: while the wave processes
        // one tile, the loads of its next kStages-1 tiles are in flight.  The
        // scheduling barriers keep each prefetch issued before the processing
        // of the current tile starts.  The loop runs whole rounds of kStages
        // tiles (one back edge, no early exit), so the set of pending loads at
        // its head is the same on entry and on every iteration; the last
        // 0..kStages-1 tiles, already in flight, are processed after it.
        // Prefetches past the end load the next piece's first tile, or
        // re-load the last tile (a cache hit), which keeps every load
        // unconditional.
        {
            auto tile_of = [&](int k) __attribute__((always_inline)) { return min(k, n_tiles - 1); };
            static_for<0, kStages - 1>([&](auto I) __attribute__((always_inline)) {
                // tile 0 may already be in buf[0], loaded by the previous piece
                if (decltype(I)::value != 0 || !pre_ok) load_tile(buf[decltype(I)::value], tile_of(decltype(I)::value));
                __builtin_amdgcn_sched_barrier(0);
            });
            const int rounds = n_tiles / kStages;
            for (int rd = 0; rd < rounds; ++rd) {
                // Step i: prefetch tile k + kStages - 1 into the buffer the
                // previous step freed, then process tile k = rd * kStages + i.
                static_for<0, kStages>([&](auto I) __attribute__((always_inline)) {
                    constexpr int i = decltype(I)::value;
                    const int k = rd * kStages + i;
                    load_ext(buf[(i + kStages - 1) % kStages], k + kStages - 1);
                    __builtin_amdgcn_sched_barrier(0);
                    compute_tile(buf[i], k);
                });
            }
            const int rem = n_tiles - rounds * kStages;
            static_for<0, kStages - 1>([&](auto I) __attribute__((always_inline)) {
                constexpr int i = decltype(I)::value;
                if (rem > i) compute_tile(buf[i], rounds * kStages + i);
            });
            // tile n_tiles went to buf[n_tiles % kStages] exactly when rem == 0
            pre_ok = next_rows > 0 && rem == 0;
        }

        // The four lane groups hold partial sums over different token rows.
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        if (first == last) {   // the piece is the whole sequence: final output
            if (live) {
                const float inv = 1.f / l_run;
                float *dst = p.out + (row0 + l16) * D + dim0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < kDpl; j += 4)
                        *(f32x4_t *)(dst + i * kDpl + j) =
                            f32x4_t{acc[j][i] * inv, acc[j + 1][i] * inv, acc[j + 2][i] * inv,
                                    acc[j + 3][i] * inv};
            }
            return;
        }
        // Partial record of piece s + item: acc [rec_heads][D], then the
        // running max [rec_heads], then the sum [rec_heads].
        float *rec = rec_base + (size_t)(s + item) * rec_stride;
        if (live) {
            float *dst = rec + l16 * D + dim0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < kDpl; j += 4)
                    *(f32x4_t *)(dst + i * kDpl + j) =
                        f32x4_t{acc[j][i], acc[j + 1][i], acc[j + 2][i], acc[j + 3][i]};
            if (lg == 0) {
                rec[p.rec_heads * D + l16] = m_run;
                rec[p.rec_heads * D + p.rec_heads + l16] = l_run;
            }
        }
    };

    // ---- Items of this workgroup (at most one when balanced). ----
    for (int item = blockIdx.x; item < items.n; item += gridDim.x) {
        const int lo = items.lo(item);
        const int hi = items.lo(item + 1);
        // The sequence s holding tile `lo`, and its first tile seg.
        int s, seg;
        if (in_lds) {
            if (!active) continue;
            // Two-level 64-way search for the first s with incl[s] > lo.
            const int bk = (S + 63) >> 6;   // <= 32
            const uint64_t m1 = __ballot(lds_incl[min(S - 1, (lane + 1) * bk - 1)] > lo);
            const int f = __builtin_ctzll(m1);
            const int i2 = min(S - 1, f * bk + lane);
            const uint64_t m2 = __ballot(lane < bk && lds_incl[i2] > lo);
            s = f * bk + __builtin_ctzll(m2);
            seg = s > 0 ? __builtin_amdgcn_readfirstlane(lds_incl[s - 1]) : 0;
        } else {
            // Running inclusive scan of the per-sequence tile counts, one chunk
            // of kThreads sequences at a time (the whole workgroup).
            int base = 0;
            for (int c0 = 0;; c0 += kThreads) {
                const int sc = c0 + threadIdx.x;
                const int n = sc < S ? tiles_of(ctx_of(sc)) : 0;
                int incl = n;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int t = __shfl_up(incl, off);
                    if (lane >= off) incl += t;
                }
                if (lane == 63) lds_red[wave] = incl;
                __syncthreads();
                int before = base, chunk_total = 0;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    before += w < wave ? lds_red[w] : 0;
                    chunk_total += lds_red[w];
                }
                incl += before;
                if (sc < S && incl - n <= lo && lo < incl) {
                    lds_found[0] = sc;
                    lds_found[1] = incl - n;
                }
                __syncthreads();
                base += chunk_total;
                if (base > lo) break;   // uniform: every thread has the same base
                __syncthreads();        // lds_red is rewritten by the next chunk
            }
            s = lds_found[0];
            seg = lds_found[1];
            __syncthreads();            // lds_found may be rewritten by the next item
            if (!active) continue;
        }
        auto seq_ctx = [&](int sq) __attribute__((always_inline)) -> int {
            return in_lds ? __builtin_amdgcn_readfirstlane(lds_ctx[sq]) : ctx_of(sq);
        };
        // Pieces of the item: the operands of the next piece are loaded
        // before the current one streams, so a piece starts without waiting
        // for its query and block ids.
        Meta mc, mn;
        pre_ok = false;
        int ctx = seq_ctx(s);
        if (ctx > 0) load_meta(mc, s, (lo - seg) * kTile, min(ctx, (hi - seg) * kTile));
        for (int x = lo; x < hi; ++s) {
            const int nt = tiles_of(ctx);
            const int end = min(hi, seg + nt);
            const int first = items.of(seg), last = items.of(seg + nt - 1);
            if (x == seg && unit == 0 && lane == 0) {   // the piece that starts the sequence
                p.seg_items[2 * s] = first;
                p.seg_items[2 * s + 1] = last;
            }
            const int ctx_next = end < hi ? seq_ctx(s + 1) : 0;
            const int next_end = min(ctx_next, (hi - end) * kTile);   // tokens of the next piece
            if (ctx_next > 0) load_meta(mn, s + 1, 0, next_end);
            process(s, ctx, x - seg, end - seg, first, last, item, mc, mn,
                    ctx_next > 0 ? min(kTile, next_end) : 0);
            if (ctx_next > 0) mc = mn;   // (an empty next sequence needs none)
            ctx = ctx_next;
            x = end;
            seg += nt;
        }
    }
}

struct MergeParams {
    const float *part;
    const int32_t *seg_items;
    float *out;
    int num_q_heads;
    int group;
    int n_chunks;
    int rec_heads;
    int max_pieces;
};

// Merge the partial records of one (sequence, query head) row whose sequence
// was split over several items: M = max_p m_p, w_p = 2^(m_p - M),
// out = sum_p w_p acc_p / sum_p w_p l_p.  Wave w takes pieces w, w + 4, ...
// in index order and merges them online (running max, rescaled sums),
// kUnroll pieces' loads in flight at a time (16 where a sequence can have
// hundreds of pieces, 4 otherwise -- more only adds latency to short
// merges; the order, hence the result, is the same); the four wave results
// are then combined in wave order, so the result does not depend on timing.
template <int D, int kUnroll>
__global__ __launch_bounds__(kThreads) void pa_merge_kernel(const MergeParams p) {
    constexpr int kPer = D / 64;   // dims per lane
    __shared__ float lds_m[kWaves], lds_l[kWaves];
    __shared__ __attribute__((aligned(16))) float lds_acc[kWaves][D];
    const int row = blockIdx.x;    // s * Hq + h
    const int s = row / p.num_q_heads;
    const int h = row - s * p.num_q_heads;
    const int first = p.seg_items[2 * s], last = p.seg_items[2 * s + 1];
    if (first == last) return;     // whole sequence: written by the decode kernel
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = h / p.group, hg = h - g * p.group;
    const int unit = g * p.n_chunks + hg / kHeads;
    const int hh = hg % kHeads;
    const size_t rec_floats = (size_t)p.rec_heads * (D + 2);
    const float *rec0 = p.part + ((size_t)(unit / kWaves) * p.max_pieces * kWaves + unit % kWaves) * rec_floats;
    const size_t stride = (size_t)kWaves * rec_floats;
    const int m_off = p.rec_heads * D + hh, l_off = p.rec_heads * D + p.rec_heads + hh;
    const int a_off = hh * D + lane * kPer;
    float M = -INFINITY, L = 0.f, a[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) a[e] = 0.f;
    for (int j0 = first + wave; j0 <= last; j0 += kUnroll * kWaves) {
        float mj[kUnroll], lj[kUnroll], aj[kUnroll][kPer];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = j0 + u * kWaves;
            const bool ok = j <= last;
            const float *r = rec0 + (size_t)(s + (ok ? j : first)) * stride;
            mj[u] = ok ? r[m_off] : -INFINITY;
            lj[u] = r[l_off];
#pragma unroll
            for (int e = 0; e < kPer; ++e) aj[u][e] = r[a_off + e];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (mj[u] == -INFINITY) continue;   // past the last piece
            const float mn = fmaxf(M, mj[u]);
            const float c = __builtin_amdgcn_exp2f(M - mn);   // 0 while M is -inf
            const float f = __builtin_amdgcn_exp2f(mj[u] - mn);
            L = fmaf(f, lj[u], L * c);
#pragma unroll
            for (int e = 0; e < kPer; ++e) a[e] = fmaf(f, aj[u][e], a[e] * c);
            M = mn;
        }
    }
    if (lane == 0) {
        lds_m[wave] = M;
        lds_l[wave] = L;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) lds_acc[wave][lane * kPer + e] = a[e];
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Mt = fmaxf(Mt, lds_m[w]);
    float Lt = 0.f, o[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(lds_m[w] - Mt);   // 0 for a wave without pieces
        Lt = fmaf(f, lds_l[w], Lt);
#pragma unroll
        for (int e = 0; e < kPer; ++e) o[e] = fmaf(f, lds_acc[w][lane * kPer + e], o[e]);
    }
    const float inv = 1.f / Lt;
#pragma unroll
    for (int e = 0; e < kPer; ++e) p.out[(size_t)row * D + lane * kPer + e] = o[e] * inv;
}

// ----------------------------------------------------------------------------
// Host side: validation, plan, dispatch.

struct Plan {
    int n_chunks;
    int units;
    int groups;       // unit groups = gridDim.y
    int item_tiles;   // 0 = balanced
    int max_pieces;   // partial records per (unit group, wave)
    int rec_heads;
    int log2_bs;
    int max_ctx;
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// Shape checks and the device-independent plan.
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
    pl->n_chunks = (group + kHeads - 1) / kHeads;
    pl->units = sh->num_kv_heads * pl->n_chunks;
    pl->groups = (pl->units + kWaves - 1) / kWaves;
    pl->rec_heads = group < kHeads ? group : kHeads;
    pl->log2_bs = ilog2(sh->block_size);
    pl->max_ctx = (int)max_ctx;
    // Upper bound of the work-list length (every sequence at max_ctx).
    const int64_t t_max = (int64_t)sh->num_seqs * ((max_ctx + kTile - 1) / kTile);
    if (t_max >= ((int64_t)1 << 31) || pl->groups > 65535) return PA_ERR_UNSUPPORTED;
    if ((int64_t)sh->num_seqs * sh->num_q_heads >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    pl->item_tiles = sh->split_tokens / kTile;
    const int64_t items = pl->item_tiles ? (t_max + pl->item_tiles - 1) / pl->item_tiles : kMaxItems;
    const int64_t pieces = (int64_t)sh->num_seqs + items;
    if (pieces * pl->groups * kWaves * pl->rec_heads * (sh->head_dim + 2) >= ((int64_t)1 << 40))
        return PA_ERR_UNSUPPORTED;
    pl->max_pieces = (int)pieces;
    return PA_OK;
}

// Workgroups of the decode kernel the current device holds at once (queried
// once per device and kernel).
template <int D, int KV>
hipError_t blocks_per_cu(int *n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, pa_decode_kernel<D, KV>, kThreads, 0);
}

// The cache entries are atomics: host threads making their first call at
// the same time may both query and store, but they store the same value.
int device_capacity(int head_dim, int kind) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev][6];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
    const int slot = (head_dim == 128 ? 3 : 0) + kind;
    std::atomic<int> &c = cache[dev][slot];
    const int known = c.load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    int per_cu = 0;
    hipError_t e;
    switch (slot) {
        case 0: e = blocks_per_cu<64, kBf16>(&per_cu); break;
        case 1: e = blocks_per_cu<64, kInt8>(&per_cu); break;
        case 2: e = blocks_per_cu<64, kFp8>(&per_cu); break;
        case 3: e = blocks_per_cu<128, kBf16>(&per_cu); break;
        case 4: e = blocks_per_cu<128, kInt8>(&per_cu); break;
        default: e = blocks_per_cu<128, kFp8>(&per_cu); break;
    }
    if (e != hipSuccess || per_cu <= 0) per_cu = 1;
    const int total = cus * per_cu;
    c.store(total, std::memory_order_relaxed);
    return total;
}

struct WsLayout {
    size_t seg_offset;
    size_t total;
};

WsLayout workspace_layout(const pa_shape *sh, const Plan &pl) {
    WsLayout w;
    const size_t rec_floats = (size_t)pl.rec_heads * (sh->head_dim + 2);
    const size_t part_bytes = (size_t)pl.groups * pl.max_pieces * kWaves * rec_floats * sizeof(float);
    w.seg_offset = (part_bytes + 255) & ~(size_t)255;
    w.total = w.seg_offset + (((size_t)sh->num_seqs * 2 * sizeof(int32_t) + 255) & ~(size_t)255);
    return w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Argument checks shared by every decode entry point, then the grid: returns
// PA_OK with *pl and *wgs (workgroups per unit group) filled, or an error.
int decode_prepare(int kind, const void *q, const void *k, const void *v, const float *ks,
                   const float *vs, const int32_t *bt, const int32_t *cl, const float *out,
                   const pa_shape *sh, Plan *pl) {
    int rc = make_plan(sh, pl);
    if (rc != PA_OK) return rc;
    if (sh->num_seqs == 0) return PA_OK;
    if (!q || !k || !v || !bt || !cl || !out) return PA_ERR_NULL;
    if (kind == kInt8 && (!ks || !vs)) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PA_ERR_ALIGNMENT;
    return PA_OK;
}

// Workgroups per unit group of the decode grid on the current device, or 0.
int decode_grid(int kind, const pa_shape *sh, const Plan &pl) {
    const int cap = device_capacity(sh->head_dim, kind);
    if (cap <= 0) return 0;
    int wgs = cap / pl.groups;
    if (wgs < 1) wgs = 1;
    if (wgs > kMaxItems) wgs = kMaxItems;
    return wgs;
}

// The decode and merge launches, with the partial records at `part` (room
// for `max_pieces` records per (unit group, wave)) and the item range of each
// sequence at `seg`.
int decode_launch(int kind, const void *q, const void *k, const void *v, const float *ks,
                  const float *vs, const int32_t *bt, const int32_t *cl, float scale, float *out,
                  const pa_shape *sh, const Plan &pl, int wgs, int max_pieces, float *part,
                  int32_t *seg, void *stream) {
    Params prm;
    prm.q = (const uint16_t *)q;
    prm.k = k;
    prm.v = v;
    prm.k_scales = ks;
    prm.v_scales = vs;
    prm.block_tables = bt;
    prm.context_lens = cl;
    prm.out = out;
    prm.part = part;
    prm.seg_items = seg;
    prm.scale_log2 = scale * kLog2e;
    prm.num_seqs = sh->num_seqs;
    prm.num_q_heads = sh->num_q_heads;
    prm.num_kv_heads = sh->num_kv_heads;
    prm.group = sh->num_q_heads / sh->num_kv_heads;
    prm.n_chunks = pl.n_chunks;
    prm.units = pl.units;
    prm.rec_heads = pl.rec_heads;
    prm.max_blocks_per_seq = sh->max_blocks_per_seq;
    prm.max_ctx = pl.max_ctx;
    prm.log2_block_size = pl.log2_bs;
    prm.item_tiles = pl.item_tiles;
    prm.max_pieces = max_pieces;
    MergeParams mp;
    mp.part = prm.part;
    mp.seg_items = prm.seg_items;
    mp.out = out;
    mp.num_q_heads = sh->num_q_heads;
    mp.group = prm.group;
    mp.n_chunks = pl.n_chunks;
    mp.rec_heads = pl.rec_heads;
    mp.max_pieces = max_pieces;
    const dim3 grid(wgs, pl.groups), block(kThreads);
    const dim3 mgrid((unsigned)((int64_t)sh->num_seqs * sh->num_q_heads));
    // fixed items that can give a sequence 64 or more pieces: more loads in flight
    const bool long_merge = pl.item_tiles > 0 && ((int64_t)pl.max_ctx + kTile - 1) / kTile >= 64LL * pl.item_tiles;
    hipStream_t st = (hipStream_t)stream;
    if (sh->head_dim == 128) {
        if (kind == kInt8) hipLaunchKernelGGL((pa_decode_kernel<128, kInt8>), grid, block, 0, st, prm);
        else if (kind == kFp8) hipLaunchKernelGGL((pa_decode_kernel<128, kFp8>), grid, block, 0, st, prm);
        else hipLaunchKernelGGL((pa_decode_kernel<128, kBf16>), grid, block, 0, st, prm);
        if (long_merge) hipLaunchKernelGGL((pa_merge_kernel<128, 16>), mgrid, block, 0, st, mp);
        else hipLaunchKernelGGL((pa_merge_kernel<128, 4>), mgrid, block, 0, st, mp);
    } else {
        if (kind == kInt8) hipLaunchKernelGGL((pa_decode_kernel<64, kInt8>), grid, block, 0, st, prm);
        else if (kind == kFp8) hipLaunchKernelGGL((pa_decode_kernel<64, kFp8>), grid, block, 0, st, prm);
        else hipLaunchKernelGGL((pa_decode_kernel<64, kBf16>), grid, block, 0, st, prm);
        if (long_merge) hipLaunchKernelGGL((pa_merge_kernel<64, 16>), mgrid, block, 0, st, mp);
        else hipLaunchKernelGGL((pa_merge_kernel<64, 4>), mgrid, block, 0, st, mp);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int decode_common(int kind, const void *q, const void *k, const void *v, const float *ks,
                  const float *vs, const int32_t *bt, const int32_t *cl, float scale, float *out,
                  const pa_shape *sh, void *ws, size_t ws_bytes, void *stream) {
    Plan pl;
    int rc = decode_prepare(kind, q, k, v, ks, vs, bt, cl, out, sh, &pl);
    if (rc != PA_OK || sh->num_seqs == 0) return rc;
    const WsLayout wl = workspace_layout(sh, pl);
    if (!ws || ws_bytes < wl.total) return PA_ERR_WORKSPACE;
    if (!aligned16(ws)) return PA_ERR_ALIGNMENT;
    const int wgs = decode_grid(kind, sh, pl);
    if (wgs <= 0) return PA_ERR_LAUNCH;
    return decode_launch(kind, q, k, v, ks, vs, bt, cl, scale, out, sh, pl, wgs, pl.max_pieces,
                         (float *)ws, (int32_t *)((char *)ws + wl.seg_offset), stream);
}

// Scratch of the allocation-free decode (paged_attn_decode_noalloc): its
// partial records and item ranges, at most kScratchBytes.
constexpr size_t kScratchBytes = (size_t)32 << 20;

}  // namespace

// The array behind kScratchBytes.  Each device the library runs on holds its
// own copy until the process ends.  In host code this name stands for a
// host-side shadow, not a device address: kernels only ever get the address
// hipGetSymbolAddress reports for the current device (scratch_address).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device with that device current and kept; nullptr if the lookup fails.
void *scratch_address() {
    constexpr int kMaxDev = 64;
    static std::atomic<void *> addr[kMaxDev];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev].store(p, std::memory_order_release);
    return p;
}

// Bytes of scratch a call needs: partial records for the pieces it can make
// (sequences + items; with the balanced split the items are at most the
// workgroups of the grid) and the item ranges, each rounded up to 256 bytes.
size_t noalloc_bytes(const pa_shape *sh, const Plan &pl, int items_upper, int *max_pieces) {
    *max_pieces = sh->num_seqs + items_upper;
    const size_t rec_floats = (size_t)pl.rec_heads * (sh->head_dim + 2);
    const size_t part = (size_t)pl.groups * (size_t)*max_pieces * kWaves * rec_floats * sizeof(float);
    return ((part + 255) & ~(size_t)255) + (((size_t)sh->num_seqs * 2 * sizeof(int32_t) + 255) & ~(size_t)255);
}

}  // namespace

extern "C" {

int paged_attn_plan(const pa_shape *shape, int32_t *split_tokens, int32_t *max_splits) {
    Plan pl;
    int rc = make_plan(shape, &pl);
    if (rc != PA_OK) return rc;
    if (split_tokens) *split_tokens = pl.item_tiles * kTile;
    if (max_splits) *max_splits = pl.max_pieces - shape->num_seqs;
    return PA_OK;
}

size_t paged_attn_workspace_bytes(const pa_shape *shape) {
    Plan pl;
    if (make_plan(shape, &pl) != PA_OK) return 0;
    return workspace_layout(shape, pl).total;
}

int paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      float *out, const pa_shape *shape, void *workspace, size_t workspace_bytes,
                      void *stream) {
    return decode_common(kBf16, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                         scale, out, shape, workspace, workspace_bytes, stream);
}

int paged_attn_decode_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                          const int32_t *block_tables, const int32_t *context_lens, float scale,
                          float *out, const pa_shape *shape, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return decode_common(kFp8, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                         scale, out, shape, workspace, workspace_bytes, stream);
}

int paged_attn_decode_int8(const void *q, const int8_t *k_cache, const int8_t *v_cache,
                           const float *k_scales, const float *v_scales,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           float *out, const pa_shape *shape, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return decode_common(kInt8, q, k_cache, v_cache, k_scales, v_scales, block_tables,
                         context_lens, scale, out, shape, workspace, workspace_bytes, stream);
}

int paged_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              float scale, float *out, const pa_shape *shape, void *stream) {
    Plan pl;
    int rc = decode_prepare(kBf16, q, k_cache, v_cache, nullptr, nullptr, block_tables,
                            context_lens, out, shape, &pl);
    if (rc != PA_OK || shape->num_seqs == 0) return rc;
    int max_pieces = 0;
    // Fixed items: their number is known from the shape alone.
    const int fixed_items = pl.item_tiles ? pl.max_pieces - shape->num_seqs : 0;
    if (fixed_items && noalloc_bytes(shape, pl, fixed_items, &max_pieces) > kScratchBytes)
        return PA_ERR_SCRATCH;
    const int wgs = decode_grid(kBf16, shape, pl);
    if (wgs <= 0) return PA_ERR_LAUNCH;
    const size_t need = noalloc_bytes(shape, pl, fixed_items ? fixed_items : wgs, &max_pieces);
    if (need > kScratchBytes) return PA_ERR_SCRATCH;
    char *base = (char *)scratch_address();
    if (!base) return PA_ERR_LAUNCH;
    const size_t seg_offset = need - (((size_t)shape->num_seqs * 2 * sizeof(int32_t) + 255) & ~(size_t)255);
    return decode_launch(kBf16, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                         scale, out, shape, pl, wgs, max_pieces, (float *)base,
                         (int32_t *)(base + seg_offset), stream);
}

const char *paged_attn_strerror(int code) {
    switch (code) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "invalid shape";
        case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size or problem size";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_LAUNCH: return "kernel launch failed or no usable device";
        case PA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case PA_ERR_SCRATCH:
            return "problem needs more than the 32 MiB static scratch of paged_attn_decode_noalloc";
        default: return "unknown error";
    }
}

int paged_attn_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
