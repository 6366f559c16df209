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
// (v_mfma_f32_16x16x32_bf16 / _f16: A 16x32, B 32x16, lane l holding row / column l%16
// and k-elements 8*(l/16) .. +7; C lane l holding column l%16, rows 4*(l/16)+i).
//
// A "row" is a (query token, query head of the kv head's group) pair.  One
// workgroup takes 256 rows of one (sequence, kv head); each of its 16 waves
// owns 16 rows (one MFMA column block).  The workgroup streams the context in
// 32-token tiles through the block table:
//   * S^T = K Q^T: K tokens are the A operand, 16 B per lane from LDS; the
//     wave's query rows are the B operand, held in registers throughout.  K
//     tiles arrive by direct-to-LDS buffer loads whose range is each
//     16-token half's valid rows, so nothing past the context end is read.
//   * causal mask and online softmax in the accumulator registers: lane l
//     holds column (row) l%16 and tokens 16 h + 4*(l/16) + i of half h.
//   * O^T += V^T P^T: the 8 weights a lane holds ARE its B-operand k-elements,
//     under the token order e -> 16*(e/4) + 4*(l/16) + e%4.
// bf16 caches: V passes through the registers of 8 waves into a dim-major
// (transposed) LDS tile as fp16 -- exact for every bf16 value below 2^16 in
// magnitude -- so the A operand is one 16-B LDS read per lane, and the
// weights enter as fp16 times 2^7 (2^-11 relative rounding; the row sums add
// the same rounded weights, and the 2^7 keeps small weights out of fp16's
// subnormals): one product per 16 dims.  A workgroup that meets a larger V
// value runs again with the tile as bf16 and the fp16 weights split exactly
// into a bf16 high part and remainder.  The tiles run in segments of four,
// one barrier each, through a ring of 8.
// FP8 caches stage K and V through registers, V as fp16 (every E4M3 value is
// one), and take the weights as fp16 likewise.  int8 caches stage K as bf16
// codes (exact); each token's V scale s = m 2^e (mantissa m in [1, 2)) is
// split: V enters as fp16 codes times 2^e (exact), the weights as fp16 with
// log2 m added to their scores (so they come out times m), and one more
// product per tile, of the weights with 1/m as an fp16 pair, gives row sums
// of the very weights each value c 2^e / (1/m) = c s is taken with -- the
// rounding cancels in the quotient as on the bf16 path.  A workgroup that
// meets a V scale outside 2^-14 .. 2^9 (other than 0) runs again with bf16
// codes and the weights times the whole scales as a bf16 pair (exact to
// 2^-17).  Both read V token-major through LDS transpose reads, one barrier
// per two tiles (FP8) or per tile (int8).
// Key split (paged_attn_prefill_split*): one chunk of one sequence is only
// (kv heads x row tiles) workgroups, a quarter of the compute units for a
// 512-token Llama-3-8B chunk, each walking ~46 tiles.  The split form cuts a
// row tile's key tiles into near-equal runs over several workgroups; each
// writes its rows' unnormalised sums with their running max and row sum, and
// a merge kernel combines the runs with log-sum-exp weights, so each row is
// still one softmax over its whole visible context (ybb.press page section
// 2.2) up to fp32 rounding order, as in the decode's merge.  A row can see no key of a
// run's first tiles (a run starting inside the causal diagonal), so its max
// starts at -inf there and its rescale factor is taken as 1.
// Scheduling: on this chip a matrix instruction holds its SIMD's vector issue
// for most of its 16 cycles (transcendentals excepted), so the vector work a
// step needs -- softmax, staging -- is as costly as its products; one step
// issues the softmax of tile i among the MFMAs of the weighted sum of tile
// i-1 and the scores of tile i+1.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "paged_prefill.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

#ifndef PF_WAVES_PER_EU
#define PF_WAVES_PER_EU 4
#endif
#ifndef PF_STAGER_PRIO
#define PF_STAGER_PRIO 3
#endif
#ifndef PF_BF16_GROUP
#define PF_BF16_GROUP 4
#endif
#ifndef PF_FP8_GROUP
#define PF_FP8_GROUP 2
#endif

#ifndef PF_WAVES
#define PF_WAVES 16
#endif
#ifndef PF_NC
#define PF_NC 1
#endif
constexpr int kWaves = PF_WAVES;           // waves per workgroup (rows share each staged tile)
constexpr int kThreads = 64 * kWaves;
constexpr int kNc = PF_NC;                 // MFMA column blocks (16 rows each) per wave
constexpr int kRowsPerWave = 16 * kNc;
constexpr int kRowsPerGroup = kRowsPerWave * kWaves;
constexpr int kTileTokens = 32;            // tokens per staged tile and step (two 16-token halves)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRsrcFlags = 0x00020000;     // word 3 of a raw buffer resource on CDNA3/CDNA4
constexpr int kWaitVmcnt0 = 0x0F70;        // s_waitcnt vmcnt(0) alone (gfx9 field layout; + n: vmcnt(n))
// Iterations run in segments of kGroup (one barrier at the end of each);
// iteration i reads K(i+1) and V(i-1) and loads K(i+kGroup+1) and
// V(i+kGroup-1), the tiles of the next segment, into a ring of 2 kGroup
// slots (slot = tile % ring): the slot a load overwrites was last read in
// the previous segment.  bf16 tiles (K straight to LDS, V^T through the
// staging waves' registers, a tile's worth in flight) take segments of four
// iterations, a quarter of the barriers; int8 / FP8 tiles come through all
// waves' registers, one tile's worth per iteration of a segment: FP8 takes
// segments of two, int8 (its registers full) segments of one.
template <int KV>
constexpr int kGroupOf = KV == 0 ? PF_BF16_GROUP : KV == 2 ? PF_FP8_GROUP : 1;

// Element kinds of the cache read: bf16, int8 codes with an fp32 scale per
// (slot, kv head), FP8 E4M3 codes.
enum KvKind : int { kBf16 = 0, kInt8 = 1, kFp8 = 2 };

struct PrefillParams {
    const uint16_t *q;
    const void *k;
    const void *v;
    const float *k_scales;   // int8: [NB, bs, Hkv]
    const float *v_scales;
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *q_offsets;
    float *out;
    float scale_log2;        // |scale| log2(e)
    uint32_t q_sign;         // 0x80008000 when scale < 0: q is negated on load
    int num_q_heads;
    int num_kv_heads;
    int group;
    int max_blocks_per_seq;
    int log2_block_size;
    int num_seqs;
    int tiles_x;             // row tiles per (sequence, kv head)
    int key_splits;          // key pieces per row tile (1: one workgroup takes all the keys)
    float *part_acc;         // key_splits > 1: unnormalised sums [units][key_splits][256][D]
    float *part_ml;          //   and (running max, row sum) pairs [units][key_splits][256][2]
};

// LDS staging of one 32-token tile of one kv head's K or V (D*2 bytes a
// token, 16-B chunks of 8 dims).  Each layout makes its operand reads
// bank-conflict free and lets a 1-KB piece of the tile arrive as one
// direct-to-LDS load of 16 B a lane.
//   K: per 16-token half, chunk-major: chunk c of token r at
//      (r / 16) * 16 * chunks + c * 16 + r % 16 (16-B units) -- the scores
//      read 16 tokens at one chunk, 256 contiguous bytes.
//   V: token-major, chunk c of token r at r * chunks + (c ^ f(r)), f(r) even
//      -- a transpose read takes 8 B (4 dims) of 16 tokens; f spreads the
//      16 tokens' 32-B dim ranges over distinct banks, 8 tokens a pass.
//   V^T (bf16 caches): dim-major, one 64-B row per dim holding the tile's 32
//      tokens as 2-B values in the weights' k-order (16-B chunk h: tokens
//      4h .. 4h+3 then 16+4h .. 16+4h+3), chunk h of row d at position
//      h ^ ((d / 2) % 4).  Measured on gfx950 (16 waves a CU, 16-B reads of
//      16 rows x 4 chunks): this swizzle reads at the contiguous rate, where
//      unswizzled 64-B or 80-B rows took 1.5x as long.
template <int D>
struct TileLds {
    static constexpr int kVtPitch = 64;
    static constexpr int kVtBytes = D * kVtPitch;
    // byte of 16-B chunk h of V^T row d
    __device__ static int vt_chunk(int d, int h) { return d * kVtPitch + 16 * (h ^ ((d >> 1) & 3)); }
    static constexpr int kChunks = D / 8;
    static constexpr int kRowBytes = D * 2;
    static constexpr int kBytes = kTileTokens * kRowBytes;            // one tensor
    static constexpr int kRowsPerBankSpan = 256 / kRowBytes;          // tokens in 256 B (one pass of banks)
    __device__ static int k_offset(int row, int chunk) {
        return (row >> 4) * (kChunks * 256) + chunk * 256 + (row & 15) * 16;
    }
    __device__ static int v_swz(int row) { return 2 * ((row / kRowsPerBankSpan) % (kChunks / 2)); }
    __device__ static int v_offset(int row, int chunk) { return row * kRowBytes + ((chunk ^ v_swz(row)) * 16); }
};

// Max over the four lane groups (lanes l, l^16, l^32, l^48) with two VALU
// lane swaps: the upper and lower 32 lanes, then the odd and even 16-lane rows.
__device__ __forceinline__ float group_max(float x) {
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Bits of the bf16 pair (x, y), x in the low half, from two floats whose low
// 16 bits are zero.
__device__ __forceinline__ uint32_t pack_hi16(float x, float y) {
    return __builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
}
// Signed byte b of w as float (exact).
__device__ __forceinline__ float i8_at(uint32_t w, int b) { return (float)(int)(int8_t)((w >> (8 * b)) & 0xffu); }

// Eight codes (8 bytes) of an int8 or FP8 E4M3 cache -> eight bf16 (16 B),
// exactly: an int8 code has at most 8 significant bits, and every E4M3 value
// (subnormals and NaN included) is a bf16 value (conversion scale 1).
template <int KV>
__device__ __forceinline__ u32x4_t codes_to_bf16x8(const u32x2_t w) {
    u32x4_t r;
    if constexpr (KV == kFp8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            r[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, false));
            r[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, true));
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            r[2 * h] = pack_hi16(i8_at(w[h], 0), i8_at(w[h], 1));
            r[2 * h + 1] = pack_hi16(i8_at(w[h], 2), i8_at(w[h], 3));
        }
    }
    return r;
}

// Eight FP8 E4M3 codes -> eight fp16 values, exactly (every E4M3 value,
// subnormals and NaN included, is an fp16 value; conversion scale 1).
__device__ __forceinline__ u32x4_t fp8x8_to_f16x8(const u32x2_t w) {
    u32x4_t r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        r[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.0f, false));
        r[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.0f, true));
    }
    return r;
}

// Eight int8 codes c -> eight fp16 values c * f, f = 2^e with -14 <= e <= 8
// (or 0), exactly: c * 2^e lies between 2^-14 and 2^15 in magnitude, normal
// fp16.  The fp16 with bits 0x64 : (c ^ 0x80) is 1024 + 128 + c.
__device__ __forceinline__ u32x4_t i8x8_to_f16x8_times(const u32x2_t w, const f16x2_t f) {
    const f16x2_t bias = f16x2_t{1152.0f16, 1152.0f16};
    u32x4_t r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t x = w[h] ^ 0x80808080u;
        // bytes (x0, 0x64, x1, 0x64) and (x2, 0x64, x3, 0x64)
        const uint32_t a = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
        const uint32_t b = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
        r[2 * h] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, a) - bias) * f);
        r[2 * h + 1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, b) - bias) * f);
    }
    return r;
}

// Dispatch order of the sequences, heaviest first.  A sequence's work is
// about its query rows times its visible context; sequences go by work
// bucket (0 for no rows, else 1 + floor(log2(rows * context)), at most 63),
// heavier buckets first, and within a bucket by index, later first.  Every
// workgroup computes the same order from the lengths; returns the sequence of
// rank r.  Batches of more than kRankSeqs sequences keep the index order
// (later first).  Workgroup-uniform; contains barriers.
constexpr int kRankSeqs = 2048;
constexpr int kRankBuckets = 64;
__device__ __forceinline__ int bucket_of(int nq, int ctx, int group) {
    const int64_t rows = (int64_t)nq * group;
    const int64_t w = rows * (int64_t)max(ctx, 0);
    if (rows <= 0 || w <= 0) return 0;
    return min(kRankBuckets - 1, 64 - __builtin_clzll((unsigned long long)w));
}
__device__ __forceinline__ int work_bucket(const PrefillParams &p, int s) {
    return bucket_of(p.q_offsets[s + 1] - p.q_offsets[s], p.context_lens[s], p.group);
}

// The sequence of rank r with its query offsets and context length.  Up to
// 64 sequences, every wave finds it on its own, without LDS or barriers:
// lane i holds sequence i's lengths and the key (bucket << 6) | i, unique and
// ordered as the dispatch order (heavier bucket, then later index, first);
// the key of rank r (r keys above it) is built bit by bit from the top, a
// bit kept when at least r + 1 keys reach the prefix.  The lengths come from
// the lanes, so they cost no second round trip.
struct SeqInfo {
    int s, q0, q1, ctx;
};
__device__ __forceinline__ SeqInfo small_batch_rank(const PrefillParams &p, int r) {
    const int lane = threadIdx.x & 63;
    const bool in = lane < p.num_seqs;
    const int qa = in ? p.q_offsets[lane] : 0;
    const int qb = in ? p.q_offsets[lane + 1] : 0;
    const int cl = in ? p.context_lens[lane] : 0;
    const int key = in ? (bucket_of(qb - qa, cl, p.group) << 6) | lane : -1;
    int ans = 0;
#pragma unroll
    for (int bit = 11; bit >= 0; --bit) {
        const int t = ans | (1 << bit);
        if (__popcll(__ballot(key >= t)) >= (unsigned)(r + 1)) ans = t;
    }
    const int sq = ans & 63;
    return {sq, __builtin_amdgcn_readlane(qa, sq), __builtin_amdgcn_readlane(qb, sq),
            __builtin_amdgcn_readlane(cl, sq)};
}

__device__ __forceinline__ int sequence_of_rank(const PrefillParams &p, int r, uint8_t *lds_b,
                                                int *lds_cnt, int *lds_sel) {
    const int S = p.num_seqs;
    if (S > kRankSeqs) return S - 1 - r;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < kRankBuckets) lds_cnt[tid] = 0;
    __syncthreads();
    for (int i = tid; i < S; i += kThreads) {
        const int b = work_bucket(p, i);
        lds_b[i] = (uint8_t)b;
        atomicAdd(&lds_cnt[b], 1);
    }
    __syncthreads();
    if (wave == 0) {
        // lane l holds bucket 63 - l: sequences of heavier buckets come first
        const int cnt = lds_cnt[kRankBuckets - 1 - lane];
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        if (incl - cnt <= r && r < incl) {
            lds_sel[0] = kRankBuckets - 1 - lane;   // the bucket of rank r
            lds_sel[1] = r - (incl - cnt);          // its place there, by index from the top
        }
    }
    __syncthreads();
    const int B = lds_sel[0];
    int k = lds_sel[1];
    __syncthreads();   // lds_cnt is reused below
    // the k-th sequence of bucket B, scanning indices downward kThreads at a time
    for (int top = S - 1; top >= 0; top -= kThreads) {
        const int i = top - tid;
        const bool in = i >= 0 && lds_b[i] == B;
        const uint64_t bal = __ballot(in);
        if (lane == 0) lds_cnt[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = lds_cnt[w];
            if (w < wave) before += c;
            total += c;
        }
        const int mine = before + __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (in && mine == k) lds_sel[0] = i;
        __syncthreads();
        if (k < total) return lds_sel[0];   // uniform: every thread has the same k and total
        k -= total;
        __syncthreads();   // lds_cnt and lds_sel are rewritten by the next pass
    }
    return S - 1 - r;   // not reached: rank r < S lies in some bucket
}

// kSplit: the key-split form (p.key_splits > 1): a workgroup takes one run of
// its row tile's key tiles.  The unsplit form compiles with run 0 of 1.
template <int D, int KV, bool kSplit>
__global__ __launch_bounds__(kThreads, PF_WAVES_PER_EU) void pa_prefill_kernel(const PrefillParams p) {
    constexpr int kSteps = D / 32;    // QK k-steps of 32 dims
    constexpr int kDpl = D / 16;      // PV output blocks of 16 dims
    using TL = TileLds<D>;
    // bf16: a K tile is loaded as 1-KB pieces, one direct-to-LDS load of 16
    // B per lane each, within one 16-token half (the piece's block-table
    // entry, and its buffer resource, are wave-uniform), by waves 0 ..
    // kPieces-1; the V tile comes through the registers of the next kVWaves
    // waves, 16 dims each, transposed (V^T).
    constexpr int kPieces = TL::kBytes / 1024;
    constexpr int kPiecesPerWave = (kPieces + kWaves - 1) / kWaves;
    static_assert(TL::kBytes % 1024 == 0 && TL::kChunks % 4 == 0, "pieces within one half");
    constexpr int kVWaves = D / 16;                      // V^T staging waves: one per 16-dim block
    constexpr int kVWave0 = kPieces + kVWaves <= kWaves ? kPieces : 0;
    static_assert(kVWave0 + kVWaves <= kWaves && kVWaves <= 8, "staging waves");
    // bf16 and FP8: the weighted sum on fp16 (V as fp16: exact for every
    // E4M3 value, and for every bf16 value of magnitude below 2^16), the
    // weights times 2^kPBias.  int8: the same weights, in both modes (the key
    // pieces of a row tile may run in different modes), also on fp16 in the
    // fast mode (below).
    constexpr bool kF16 = KV == kFp8 || KV == kBf16;
    constexpr float kPBias = 7.f;
    constexpr int kGroup = kGroupOf<KV>;
    constexpr int kRing = 2 * kGroup;
    constexpr bool kVt = KV == kBf16;     // V staged transposed (V^T), as fp16
    __shared__ __attribute__((aligned(1024))) char lds_k[kRing][TL::kBytes];
    __shared__ __attribute__((aligned(1024))) char lds_v[kRing][kVt ? TL::kVtBytes : TL::kBytes];   // fp16 V^T, or bf16 / fp16 V
    // Set by a wave, in its own slot, when it met a value the fast mode does
    // not hold: bf16 V beyond fp16 (see vstage_store), an int8 V scale out of
    // the fast range (see qstore)
    __shared__ int lds_wide[kWaves];
    __shared__ int lds_pmax[kWaves];
    __shared__ uint8_t lds_rank_b[kRankSeqs];
    __shared__ int lds_rank_cnt[kWaves > kRankBuckets ? kWaves : kRankBuckets];
    __shared__ int lds_rank_sel[2];
    // int8: per token of the kv head, stored with the K tile (see qstore):
    // its K scale [0] and, fast mode, log2 of its V scale's mantissa over c
    // [1]; and its V scale, two tiles before its V tile, in a ring of four
    // (read until the weighted sum of its tile, an iteration after that tile)
    __shared__ __attribute__((aligned(16))) float lds_sc[KV == kInt8 ? 2 : 1][kRing][kTileTokens];
    constexpr int kVsRing = 4;
    __shared__ __attribute__((aligned(16))) float lds_vs[KV == kInt8 ? kVsRing : 1][kTileTokens];
    // int8 fast mode: the A operand of the row-sum product (see
    // weighted_values): row 0 the V scale mantissas' reciprocals rounded to
    // fp16, row 1 the remainder times 2^10, rows 2..15 zero; [slot][row]
    // [lane group][k-element]
    __shared__ __attribute__((aligned(16))) _Float16 lds_rs[KV == kInt8 ? kRing : 1][16][4][8];

    // Workgroup L runs on XCD L % 8 (round-robin dispatch).  (sequence, kv
    // head) pair P -- heaviest sequences first -- goes to XCD P % 8, and an
    // XCD runs its pairs in order, all row tiles of a pair together, so the
    // row tiles that read the same K/V share one L2.
    // With key pieces, a row tile's pieces are consecutive workgroups of its XCD.
    const int xcd = (int)(blockIdx.x % 8);
    const int y = (int)(blockIdx.x / 8);
    const int splits = kSplit ? p.key_splits : 1;
    const int per_pair = p.tiles_x * splits;
    const int P = (y / per_pair) * 8 + xcd;
    if (P >= p.num_kv_heads * p.num_seqs) return;    // uniform: the whole workgroup
    SeqInfo si;
    if (p.num_seqs <= 64) {
        si = small_batch_rank(p, P / p.num_kv_heads);
    } else {
        si.s = sequence_of_rank(p, P / p.num_kv_heads, lds_rank_b, lds_rank_cnt, lds_rank_sel);
        si.q0 = p.q_offsets[si.s];
        si.q1 = p.q_offsets[si.s + 1];
        si.ctx = p.context_lens[si.s];
    }
    const int s = si.s;
    const int g = P % p.num_kv_heads;
    const int bx = p.tiles_x - 1 - (y % per_pair) / splits;
    const int piece = (y % per_pair) % splits;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int hgrp = lane >> 4;       // lane group: k-elements / accumulator rows
    const int l16 = lane & 15;
    const int G = p.group;
    const int q0 = si.q0;
    const int nq = si.q1 - q0;
    const int R = nq * G;
    if (bx * kRowsPerGroup >= R) return;             // uniform: no row of the workgroup exists
    const int row0 = bx * kRowsPerGroup + wave * kRowsPerWave;
    const bool wave_live = row0 < R;
    const int ctx = si.ctx;
    const int Hq = p.num_q_heads;
    const int Hkv = p.num_kv_heads;
    constexpr int kElem = KV == kBf16 ? 2 : 1;             // bytes per cache element
    const uint32_t rb32 = (uint32_t)(Hkv * D * kElem);     // bytes of one token slot (all kv heads)
    const char *kbase = (const char *)p.k + (int64_t)g * D * kElem;
    const char *vbase = (const char *)p.v + (int64_t)g * D * kElem;
    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const int bs_log2 = p.log2_block_size;
    const int bs_mask = (1 << bs_log2) - 1;
    const float c = p.scale_log2;      // |scale| log2(e); a negative scale negates q
    // int8 fast mode: 1 / c (see qstore), if c is within 2^-100 .. 2^100
    const bool i8_fast_ok = KV == kInt8 && c >= 0x1p-100f && c <= 0x1p100f;
    const float inv_c = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __builtin_amdgcn_rcpf(c))));

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
            u32x4_t w = *(const u32x4_t *)(qrow + 32 * st + 8 * hgrp) ^ p.q_sign;
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
    pmax = __builtin_amdgcn_readfirstlane(pmax);      // wave-uniform after the reduction
    pmin = __builtin_amdgcn_readfirstlane(pmin);
    // The workgroup's last position.  bf16 and int8: its last row's
    // (positions grow with the row), with no barrier, so the block-table
    // window loads right after the q loads.  FP8: the waves' maxima through
    // LDS (without the barrier its kernel spills).
    int wg_pmax;
    if constexpr (kVt || KV == kInt8) {
        if (lane == 0) lds_wide[wave] = 0;
        if constexpr (KV == kInt8) {
            constexpr int kRsChunks = (int)sizeof(lds_rs) / 16;
            if ((int)threadIdx.x < kRsChunks) ((u32x4_t *)&lds_rs[0][0][0][0])[threadIdx.x] = u32x4_t{0u, 0u, 0u, 0u};
        }
        wg_pmax = ctx - nq + (min(R, (bx + 1) * kRowsPerGroup) - 1) / G;
    } else {
        if (lane == 0) {
            lds_pmax[wave] = wave_live ? pmax : -1;
            lds_wide[wave] = 0;
        }
        if constexpr (KV == kInt8) {
            constexpr int kRsChunks = (int)sizeof(lds_rs) / 16;
            if ((int)threadIdx.x < kRsChunks) ((u32x4_t *)&lds_rs[0][0][0][0])[threadIdx.x] = u32x4_t{0u, 0u, 0u, 0u};
        }
        __syncthreads();
        wg_pmax = lds_pmax[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) wg_pmax = max(wg_pmax, lds_pmax[w]);
    }
    // The row tile's tiles 0 .. n_full-1 are cut into `pieces` near-equal
    // runs; this workgroup takes run `piece`, tiles t_lo .. t_hi-1 (uniform).
    // Below, tile indices count from t_lo and tok0 is its first token.
    const int n_full = wg_pmax / kTileTokens + 1;
    const int pieces = kSplit ? max(1, min(p.key_splits, n_full)) : 1;
    if (kSplit && piece >= pieces) return;             // uniform: a short context has fewer pieces
    const int t_lo = kSplit ? piece * n_full / pieces : 0;
    const int t_hi = kSplit ? (piece + 1) * n_full / pieces : n_full;
    const int n_tiles = t_hi - t_lo;                   // the workgroup's tiles
    const int tok0 = t_lo * kTileTokens;
    // this wave's tiles: those up to its last row's position (none when that
    // lies before the run)
    const int my_steps = !kSplit || pieces == 1 ? pmax / kTileTokens + 1
                                                : min(max(pmax / kTileTokens + 1, t_lo), t_hi) - t_lo;

    // ---- bf16 K tile loads: this wave's pieces, piece index w + j * kWaves;
    // during iteration i they load tile i + kGroup + 1.
    auto piece_ok = [&](int j) __attribute__((always_inline)) {
        return kPieces % kWaves == 0 || wave + j * kWaves < kPieces;
    };
    auto piece_sub = [&](int j) __attribute__((always_inline)) { return (wave + j * kWaves) % kPieces; };
    auto piece_half = [&](int j) __attribute__((always_inline)) { return piece_sub(j) / (TL::kChunks / 4); };
    // Block-table window: lane l holds entry wbase + l, the next 64 entries
    // are loaded when the window slides (64 blocks ahead of their use), and a
    // tile's blocks are read from a lane (v_readlane), not from memory: a
    // load between a tile's K/V loads and their use would wait for them too.
    const int nblk = ((min(ctx, tok0 + n_tiles * kTileTokens) - 1) >> bs_log2) + 1;   // entries read
    auto load_window = [&](int base) __attribute__((always_inline)) {
        const int e = base + lane;
        return e < nblk ? table[e] : 0;
    };
    int wbase = 0, win = 0, win_next = 0;   // set by each pass (run)
    // physical block of token tb (0 past the context end)
    auto phys_at = [&](int tb) __attribute__((always_inline)) {
        if (tb >= ctx) return 0;
        const int o = (tb >> bs_log2) - wbase;            // 0 <= o < 128 (see the slide below)
        int b;
        if (o < 64) b = __builtin_amdgcn_readlane(win, o);
        else b = __builtin_amdgcn_readlane(win_next, o - 64);
        return b;
    };
    auto phys_of = [&](int tile, int j) __attribute__((always_inline)) {
        return phys_at(tok0 + tile * kTileTokens + 16 * piece_half(j));
    };
    // One direct-to-LDS load of 16 B a lane: the rows of the 16-token half
    // starting at token tb (physical block phys) of `base` (K or V of the kv
    // head), at byte voff of the half; lane l's 16 B land at dst + 16 l.
    auto direct_load = [&](const char *base, int tb, int phys, int voff, char *dst) __attribute__((always_inline)) {
        const int rows = min(16, max(0, ctx - tb));      // the buffer range: nothing past the context
        const int64_t slot0 = ((int64_t)phys << bs_log2) + (tb & bs_mask);
        const uint64_t addr = (uint64_t)(uintptr_t)(base + slot0 * rb32);
        // wave-uniform by construction; stated, so the resource is built in
        // scalar registers without a per-lane loop
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        const int range = __builtin_amdgcn_readfirstlane(rows * (int)rb32);
        // raw buffer resource: base, stride 0, num_records = range
        const i32x4_t rs = {(int32_t)lo, (int32_t)(hi & 0xffffu), range, kRsrcFlags};
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)dst);
        // Direct-to-LDS load (lane l's 16 B land at dst + 16 l).  Written as
        // asm so the compiler does not order LDS reads of the other ring
        // slots after it (it cannot tell the slots apart and would wait for
        // the load): the explicit waits and barriers order the slots.  M0 is
        // an input operand, so the compiler writes it and knows what it holds;
        // the nops cover the SGPR / M0 writes read by the load.
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "{m0}"(m0), "v"(voff), "s"(rs)
                     : "memory");
    };
    auto issue = [&](int tile, int j, int phys) __attribute__((always_inline)) {
        const int sub = piece_sub(j);
        // the lane's 16 B: 4 chunks x 16 tokens of one half (chunk
        // 4 (sub % (chunks/4)) + lane / 16, token lane % 16)
        const int r16 = lane & 15;
        const int chunk = 4 * (sub % (TL::kChunks / 4)) + (lane >> 4);
        const int voff = (int)((uint32_t)r16 * rb32 + (uint32_t)(chunk * 16));
        direct_load(kbase, tok0 + tile * kTileTokens + 16 * piece_half(j), phys, voff,
                    lds_k[tile % kRing] + sub * 1024);
    };

    // ---- int8 / FP8 tiles come through registers: each thread loads 8 codes
    // (8 B) of one token of a K or V tile, load number tid + jj * threads
    // (K loads first), for each tile of the next segment (one register set a
    // tile) at the end of a segment, and at the end of the next segment
    // writes them into the same LDS layouts, as bf16 (FP8 V and int8 V in the
    // fast mode: as fp16; int8 scales go to lds_sc and lds_vs), so the loads
    // have a whole segment to land.
    // 8-B code loads per thread per iteration (K + V): 8 D per tile over the
    // workgroup; with more threads than loads (D = 64) the later waves load
    // nothing (qload_ok, wave-uniform).
    constexpr int kQLoads = 8 * D / kThreads > 0 ? 8 * D / kThreads : 1;
    constexpr int kCodeChunks = D / 8;                   // 8-code chunks per token
    // one set of registers per tile of a segment (int8 / FP8; set g holds
    // the loads of the segment's g-th K and V tiles)
    constexpr int kSets = KV == kBf16 ? 1 : kGroup;
    u32x2_t st_codes[kSets][kQLoads];
    float st_scale[kSets][kQLoads];
    float st_vscale[kSets][kQLoads];    // int8, K loads: the token's V scale
    // keys and values read: the workgroup's tiles, within the context
    const int kv_end = min(ctx, tok0 + n_tiles * kTileTokens);
    // K or V: wave-uniform (4 D loads per tile and kind, a multiple of 64)
    auto qload_ok = [&](int jj) __attribute__((always_inline)) {
        return wave * 64 + jj * kThreads < 8 * D;
    };
    auto qload_is_v = [&](int jj) __attribute__((always_inline)) {
        return (wave * 64 + jj * kThreads) >= 4 * D;
    };
    // V: a wave's 64 loads are 64 / kCodeChunks whole tokens (one LDS row
    // each); K: 16 tokens of one half by 4 chunks, so each 16 lanes store
    // one 256 B run of the chunk-major layout (whole tokens there would put
    // a token's chunks, 256 B apart, in the same banks).
    constexpr int kChunkGroups = kCodeChunks / 4;        // K: 4-chunk groups per half
    auto qload_wpart = [&](int jj) __attribute__((always_inline)) {   // wave-uniform
        return ((wave * 64 + jj * kThreads) % (4 * D)) / 64;
    };
    auto qload_token = [&](int jj) __attribute__((always_inline)) {
        if (qload_is_v(jj)) return (((int)threadIdx.x + jj * kThreads) % (4 * D)) / kCodeChunks;
        return 16 * (qload_wpart(jj) / kChunkGroups) + (lane & 15);
    };
    auto qload_chunk = [&](int jj) __attribute__((always_inline)) {
        if (qload_is_v(jj)) return (((int)threadIdx.x + jj * kThreads) % (4 * D)) % kCodeChunks;
        return 4 * (qload_wpart(jj) % kChunkGroups) + (lane >> 4);
    };
    // the 16-token half of load jj, wave-uniform
    auto qload_half = [&](int jj) __attribute__((always_inline)) {
        if (qload_is_v(jj)) return (qload_wpart(jj) * 64 / kCodeChunks) >> 4;
        return qload_wpart(jj) / kChunkGroups;
    };
    auto make_rsrc = [&](const void *base, int range) __attribute__((always_inline)) {
        const uint64_t addr = (uint64_t)(uintptr_t)base;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(((uint64_t)hi << 32) | lo), 0,
                                                 __builtin_amdgcn_readfirstlane(range), kRsrcFlags);
    };
    auto qissue = [&](int tile, int jj, int set, int phys, auto safe) __attribute__((always_inline)) {
        const bool is_v = qload_is_v(jj);
        const int tb = tok0 + tile * kTileTokens + 16 * qload_half(jj);
        const int rows = min(16, max(0, kv_end - tb));   // none past the tiles or the context is read
        const int64_t slot0 = ((int64_t)phys << bs_log2) + (tb & bs_mask);
        const int r16 = qload_token(jj) & 15;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((is_v ? vbase : kbase) + slot0 * rb32, rows * (int)rb32);
        st_codes[set][jj] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
            rs, (int)((uint32_t)r16 * rb32 + (uint32_t)(qload_chunk(jj) * 8)), 0, 0));
        // int8: the tile's K and V scales, loaded (every lane of a token, one
        // dword line a wave) by the K wave of each half that holds chunk 0,
        // the one that stores them (see qstore)
        if constexpr (KV == kInt8) {
            if (!is_v && qload_wpart(jj) % kChunkGroups == 0) {
                const int64_t so = slot0 * Hkv + g;
                const __amdgpu_buffer_rsrc_t ks = make_rsrc(p.k_scales + so, rows * Hkv * 4);
                const __amdgpu_buffer_rsrc_t vs = make_rsrc(p.v_scales + so, rows * Hkv * 4);
                st_scale[set][jj] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ks, r16 * Hkv * 4, 0, 0));
                st_vscale[set][jj] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vs, r16 * Hkv * 4, 0, 0));
            }
        }
    };
    // tile `tile` of load jj; past the tiles the codes read as 0
    auto qissue_tile = [&](int tile, int jj, int set, auto safe) __attribute__((always_inline)) {
        qissue(tile, jj, set, phys_at(tok0 + tile * kTileTokens + 16 * qload_half(jj)), safe);
    };
    // int8, fast mode: a V scale s = m 2^e (mantissa m in [1, 2)) multiplies
    // the codes by 2^e in the fp16 V tile; the weights take m through their
    // scores (lds_sc[1] = log2(m) / c), and the row sums 1/m through lds_rs
    // (stored with the V tile).  A zero scale gives V = 0 and m = 1.  A scale
    // neither 0 nor within 2^-14 <= s < 2^9 (negative, tiny, huge or not
    // finite) sets the wave's lds_wide flag, and the workgroup then runs
    // again in the safe mode: V as bf16 codes, the weights times the whole
    // scales as a bf16 pair.  Register set `set` holds K tile ktile or V tile
    // vtile (whose scales are in lds_vs since the K tile two before), each
    // stored into its ring slot.
    auto mantissa = [](float sc) __attribute__((always_inline)) {
        return __uint_as_float((__float_as_uint(sc) & 0x007fffffu) | 0x3f800000u);
    };
    auto qstore = [&](int jj, int set, int ktile, int vtile, auto safe) __attribute__((always_inline)) {
        constexpr bool kI8Fast = KV == kInt8 && !decltype(safe)::value;
        const int tok = qload_token(jj), ch = qload_chunk(jj);
        const auto &codes = st_codes[set][jj];
        if (qload_is_v(jj)) {
            const int slot = vtile % kRing;
            u32x4_t val;
            if constexpr (kI8Fast) {
                const float sv = lds_vs[KV == kInt8 ? vtile % kVsRing : 0][tok];
                const uint32_t sb = __float_as_uint(sv);
                const _Float16 p2 = (_Float16)__uint_as_float(sb & 0x7f800000u);   // 2^e (or 0), exact
                val = i8x8_to_f16x8_times(codes, f16x2_t{p2, p2});
                if (ch == 0) {
                    // k-element 4 (tok / 16) + tok % 4 of lane group (tok % 16) / 4
                    const float r = __builtin_amdgcn_rcpf(mantissa(sv));
                    const _Float16 rh = (_Float16)r;
                    _Float16 *at = &lds_rs[slot][0][(tok & 15) >> 2][4 * (tok >> 4) + (tok & 3)];
                    at[0] = rh;
                    at[4 * 8] = (_Float16)((r - (float)rh) * 1024.f);     // row 1
                }
            } else {
                val = kF16 ? fp8x8_to_f16x8(codes) : codes_to_bf16x8<KV>(codes);
            }
            *(u32x4_t *)(lds_v[slot] + TL::v_offset(tok, ch)) = val;
        } else {
            const int slot = ktile % kRing;
            *(u32x4_t *)(lds_k[slot] + TL::k_offset(tok, ch)) = codes_to_bf16x8<KV>(codes);
            if constexpr (KV == kInt8) {
                if (ch == 0) {
                    const float vsc = st_vscale[set][jj];
                    lds_sc[0][slot][tok] = st_scale[set][jj];
                    lds_vs[KV == kInt8 ? ktile % kVsRing : 0][tok] = vsc;
                    if constexpr (kI8Fast) {
                        const uint32_t sb = __float_as_uint(vsc);
                        const bool fast = sb == 0u || (sb >= 0x38800000u && sb < 0x44000000u);
                        if (!fast) lds_wide[wave] = 1;
                        lds_sc[KV == kInt8 ? 1 : 0][slot][tok] = __builtin_amdgcn_logf(mantissa(vsc)) * inv_c;
                    }
                }
            }
        }
    };

    // ---- bf16 V^T staging.  Staging wave w takes the 16-token half w % 2 and
    // dims 32 (w / 2) .. + 31 of a tile; its lane l the tokens 2 p, 2 p + 1
    // of the half (p = l % 8) and dims 4 q .. 4 q + 3 of those (q = l / 8):
    // two 8-B loads, issued at the start of an iteration, written at its end
    // as four 4-B V^T runs (one per dim, its 2 tokens).  The values are
    // written as fp16; a value beyond fp16 (magnitude >= 2^16, or infinite)
    // sets the wave's lds_wide flag, and the workgroup then runs again in the safe mode,
    // which writes them as bf16.  Tokens past the context read as 0 (the
    // buffer range).
    const bool v_stager = kVt && wave >= kVWave0 && wave < kVWave0 + kVWaves;   // wave-uniform
    // The staging waves carry the most work per tile; issued first (wave
    // priority 3 of 0..3), they reach each barrier no later than the K
    // waves, which fill the SIMD's remaining issue slots.
    if (v_stager) __builtin_amdgcn_s_setprio(PF_STAGER_PRIO);
    const int vs_w = v_stager ? wave - kVWave0 : 0;
    const int vs_half = vs_w & 1;
    const int vs_p = lane & 7, vs_q = lane >> 3;
    const int vs_dim = 32 * (vs_w >> 1) + 4 * vs_q;          // the lane's first dim
    // Bytes, within a V^T slot, of the lane's two writes for dims vs_dim, +1
    // and vs_dim + 2, +3: tokens 2 p, 2 p + 1 of half h sit at byte
    // 8 h + 4 (p % 2) of chunk p / 2 (two chunk swizzles).  Opaque lane
    // constants, so each write address is one add to the slot's base.
    int vs_off01 = TL::vt_chunk(vs_dim, vs_p >> 1) + 8 * vs_half + 4 * (vs_p & 1);
    int vs_off23 = TL::vt_chunk(vs_dim + 2, vs_p >> 1) + 8 * vs_half + 4 * (vs_p & 1);
    __asm__ volatile("" : "+v"(vs_off01), "+v"(vs_off23));
    u32x2_t vst[2];
    auto vstage_issue = [&](int tile) __attribute__((always_inline)) {
        const int tb = tok0 + tile * kTileTokens + 16 * vs_half;
        const int rows = min(16, max(0, ctx - tb));
        const int64_t slot0 = ((int64_t)phys_at(tb) << bs_log2) + (tb & bs_mask);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(vbase + slot0 * rb32, rows * (int)rb32);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            vst[e] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                rs, (int)((uint32_t)(2 * vs_p + e) * rb32 + (uint32_t)(2 * vs_dim)), 0, 0));
    };
    auto vstage_store = [&](int slot, auto safe) __attribute__((always_inline)) {
        constexpr bool kSafe = decltype(safe)::value;
        // (opaque: keeps the conversion below inside the staging waves' branch)
        __asm__ volatile("" : "+v"(vst[0]), "+v"(vst[1]));
        char *row01 = lds_v[slot] + vs_off01;
        char *row23 = lds_v[slot] + vs_off23;
        auto at = [&](int k) __attribute__((always_inline)) {
            return (uint32_t *)((k < 2 ? row01 : row23) + (k & 1) * TL::kVtPitch);
        };
        if constexpr (kSafe) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *at(k) = __builtin_amdgcn_perm(vst[1][k >> 1], vst[0][k >> 1], (k & 1) ? 0x07060302u : 0x05040100u);
            return;
        }
        float f[2][4];     // [token e][dim k]
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            f[e][0] = __uint_as_float(vst[e][0] << 16);
            f[e][1] = __uint_as_float(vst[e][0] & 0xffff0000u);
            f[e][2] = __uint_as_float(vst[e][1] << 16);
            f[e][3] = __uint_as_float(vst[e][1] & 0xffff0000u);
        }
        // max magnitude (a NaN is skipped: fp16 keeps it), as three-input
        // maxima with absolute-value modifiers: written with fmaxf / fabsf the
        // compiler first quiets each input, 11 instructions instead of 4
        float m0, m1, m2, mx;
        asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m0) : "v"(f[0][0]), "v"(f[0][1]), "v"(f[0][2]));
        asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m1) : "v"(f[0][3]), "v"(f[1][0]), "v"(f[1][1]));
        asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(m2) : "v"(f[1][2]), "v"(f[1][3]), "v"(m0));
        asm("v_max_f32 %0, %1, %2" : "=v"(mx) : "v"(m1), "v"(m2));
        if (__ballot(mx >= 65536.f) != 0 && lane == 0) lds_wide[wave] = 1;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *at(k) = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{f[0][k], f[1][k]}, f16x2_t));
    };

    // ---- S^T = K Q^T of one tile from LDS: lane l gets column (row) l%16 of
    // block cb and tokens 16 bb + 4 (l/16) + i.  The k-step loop is outermost,
    // so the 2 kNc accumulation chains interleave.  int8: times the tokens' K
    // scales (the K tile holds the codes).
    typedef f32x4_t Scores[2][kNc];
    // int8 fast mode: plus log2 of the token's V scale mantissa over c, so
    // that its weight comes out times that mantissa.
    auto scores = [&](const char *kl, const float *ksc, Scores &S, auto safe) __attribute__((always_inline)) {
        bf16x8_t kop[2][kSteps];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int st = 0; st < kSteps; ++st)
                kop[bb][st] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(kl + TL::k_offset(16 * bb + l16, 4 * st + hgrp)));
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int cb = 0; cb < kNc; ++cb)
                    S[bb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        kop[bb][st], qop[cb][st], st == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : S[bb][cb], 0, 0, 0);
        if constexpr (KV == kInt8) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const f32x4_t ks = *(const f32x4_t *)(ksc + 16 * bb + 4 * hgrp);
                if constexpr (!decltype(safe)::value) {
                    // lds_sc[1] of the same slot
                    const f32x4_t lm = *(const f32x4_t *)(ksc + kRing * kTileTokens + 16 * bb + 4 * hgrp);
#pragma unroll
                    for (int cb = 0; cb < kNc; ++cb) S[bb][cb] = S[bb][cb] * ks + lm;
                } else {
#pragma unroll
                    for (int cb = 0; cb < kNc; ++cb) S[bb][cb] *= ks;
                }
            }
        }
    };

    f32x4_t acc[kDpl][kNc];               // set by each pass (run)
    float m_run[kNc], l_run[kNc];
    // int8 fast mode: the row-sum product's accumulators (lanes 0..15: row
    // sum = [0] + 2^-10 [1] of their row), rescaled with acc
    f32x4_t acc_rs[kNc];

    // ---- online softmax of tile t's scores S into the weights (bf16 high
    // part and remainder, both rounded to nearest even: hi + lo is the fp32
    // weight to 2^-17; FP8 and int8 fast mode: fp16 times 2^kPBias; int8 safe
    // mode: fp32, split with the V scales in the weighted sum), masked on the
    // tiles that cross a row's position.  The running max moves only when a row's tile max exceeds it
    // by more than 8 (log2 units): weights stay <= 2^(8 + kPBias) <= 2^15 and
    // the accumulators are rarely rescaled.  Returns whether any row of the wave moved; alpha[cb] is then
    // log2 of that row's rescale factor (0 where it did not move).
    typedef bf16x8_t Weights[kNc];
    // the 8 weights as a bf16 high part plus a bf16 remainder, both rounded
    // to nearest even: hi + lo is the fp32 weight to 2^-17
    auto split_weights = [&](const float (&pr)[8], bf16x8_t &hi8, bf16x8_t &lo8) __attribute__((always_inline)) {
        u32x4_t pw, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x2_t w2 = f32x2_t{pr[2 * e], pr[2 * e + 1]};
            const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(w2, bf16x2_t));
            const f32x2_t r2 = w2 - f32x2_t{__uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
            pw[e] = hi;
            pl[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2_t));
        }
        hi8 = __builtin_bit_cast(bf16x8_t, pw);
        lo8 = __builtin_bit_cast(bf16x8_t, pl);
    };
    auto softmax = [&](const int t, const Scores &S, Weights &Phi, Weights &Plo, float (&alpha)[kNc],
                       auto masked, auto safe) __attribute__((always_inline)) {
        constexpr bool kMasked = decltype(masked)::value;
        constexpr bool kI8Fast = KV == kInt8 && !decltype(safe)::value;
        const int t0 = tok0 + t * kTileTokens;
        bool vis[kNc][8];
        float mx[kNc];
        bool exceed = false;
#pragma unroll
        for (int cb = 0; cb < kNc; ++cb) {
            mx[cb] = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                vis[cb][e] = !kMasked || t0 + 16 * (e >> 2) + 4 * hgrp + (e & 3) <= pos[cb];
                mx[cb] = fmaxf(mx[cb], vis[cb][e] ? S[e >> 2][cb][e & 3] : -INFINITY);
            }
            exceed = exceed || mx[cb] * c > m_run[cb] + 8.f;
        }
        // Only when one of the lane's scores passes its row's running max by
        // more than 8 are the row maxima (over the four lane groups) needed.
        const bool grow = __ballot(exceed) != 0;
        if (grow) {
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                const float mt = group_max(mx[cb]) * c;       // -inf: nothing visible
                const float m_new = mt > m_run[cb] + 8.f ? mt : m_run[cb];
                // log2 of the rescale; 0 if unmoved -- also for a row that has
                // seen no key yet (a key run that starts past its position),
                // whose max stays -inf
                // (unsplit: every row sees token 0 in its first tile)
                alpha[cb] = !kSplit ? m_run[cb] - m_new : m_new > m_run[cb] ? m_run[cb] - m_new : 0.f;
                if constexpr (!kI8Fast) l_run[cb] *= __builtin_amdgcn_exp2f(alpha[cb]);
                m_run[cb] = m_new;
            }
        }
#pragma unroll
        for (int cb = 0; cb < kNc; ++cb) {
            float pr[8], psum = 0.f;
            const float nm = kPBias - m_run[cb];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e >> 2][cb][e & 3], c, nm));
                pr[e] = vis[cb][e] ? w : 0.f;
                if constexpr (!kF16 && !kI8Fast) psum += pr[e];
            }
            if constexpr (kI8Fast) {
                // fp16 weights (their scores carry the V scale mantissas); the
                // row sums come from the weighted sums' extra product
                u32x4_t pw;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pw[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{pr[2 * e], pr[2 * e + 1]}, f16x2_t));
                Phi[cb] = __builtin_bit_cast(bf16x8_t, pw);
                Plo[cb] = bf16x8_t{};
            } else if constexpr (kF16) {
                // the row sum adds the weights as rounded to fp16, the values
                // the weighted sum multiplies: their rounding then cancels in
                // the quotient where one weight dominates
                // (each pair in its own f16x2 variable: a bit_cast of a vector
                // element feeding fdot2 was compiled as element 0 every time)
                f16x2_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hv[e] = __builtin_convertvector(f32x2_t{pr[2 * e], pr[2 * e + 1]}, f16x2_t);
                    psum = __builtin_amdgcn_fdot2(hv[e], f16x2_t{1.0f16, 1.0f16}, psum, false);
                }
                Phi[cb] = __builtin_bit_cast(bf16x8_t, u32x4_t{__builtin_bit_cast(uint32_t, hv[0]), __builtin_bit_cast(uint32_t, hv[1]),
                                                             __builtin_bit_cast(uint32_t, hv[2]), __builtin_bit_cast(uint32_t, hv[3])});
                Plo[cb] = bf16x8_t{};
            }
            if constexpr (!kI8Fast) l_run[cb] += psum;
            if constexpr (kI8Fast) {
                // weights packed above
            } else if constexpr (KV == kInt8) {
                // fp32 weights, split once the V scales are in LDS (next step)
                Phi[cb] = __builtin_bit_cast(bf16x8_t, f32x4_t{pr[0], pr[1], pr[2], pr[3]});
                Plo[cb] = __builtin_bit_cast(bf16x8_t, f32x4_t{pr[4], pr[5], pr[6], pr[7]});
            } else if constexpr (kF16) {
                // weights packed above
            } else {
                split_weights(pr, Phi[cb], Plo[cb]);
            }
        }
        return grow;
    };
    auto rescale = [&](const float (&alpha)[kNc], auto safe) __attribute__((always_inline)) {
        float f[kNc];
#pragma unroll
        for (int cb = 0; cb < kNc; ++cb) f[cb] = __builtin_amdgcn_exp2f(alpha[cb]);
#pragma unroll
        for (int j = 0; j < kDpl; ++j)
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) acc[j][cb] *= f[cb];
        if constexpr (KV == kInt8 && !decltype(safe)::value)
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) acc_rs[cb] *= f[cb];
    };

    // ---- O^T += V^T P^T for one tile.  The A operand of output block j
    // (dims 16 j .. +15) is read transposed from the token-major V tile: in a
    // lane group, lane i names 4 dims (16 j + 4 (i % 4) ..) of token
    // 4 (group) + i / 4 (and 16 tokens further for the second read), and
    // gets dim 16 j + i of the group's 4 tokens -- its k-elements in the
    // weights' token order.
    const int tr_tok = 4 * hgrp + (l16 >> 2);
    const int tr_lane = tr_tok * TL::kRowBytes + 8 * (l16 & 1);   // + chunk position
    // V^T (bf16 caches): lane (group h, row i) reads 16 B of dim row 16 j + i
    // -- its 8 tokens in the weights' order -- at a fixed offset per j.
    const int vt_lane = TL::vt_chunk(l16, hgrp);   // row 16 j + i: the same swizzle as row i
    // Safe mode (bf16 V^T): the fp16 weights enter as a bf16 high part plus
    // remainder, both exact (11 significant bits).
    auto weighted_values_vt = [&](const char *vl, const Weights &Pin, auto safe) __attribute__((always_inline)) {
        constexpr bool kSafe = decltype(safe)::value;
        Weights Bhi, Blo;
        if constexpr (kSafe) {
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                const f16x8_t h = __builtin_bit_cast(f16x8_t, Pin[cb]);
                float pr[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = (float)h[e];
                split_weights(pr, Bhi[cb], Blo[cb]);
            }
        }
#pragma unroll
        for (int j = 0; j < kDpl; ++j) {
            const u32x4_t vop = *(const u32x4_t *)(vl + vt_lane + j * 16 * TL::kVtPitch);
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                if constexpr (kSafe) {
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vop), Bhi[cb],
                                                                         acc[j][cb], 0, 0, 0);
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vop), Blo[cb],
                                                                         acc[j][cb], 0, 0, 0);
                } else {
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(f16x8_t, vop), __builtin_bit_cast(f16x8_t, Pin[cb]), acc[j][cb], 0, 0, 0);
                }
            }
        }
    };
    // int8: fast mode, the weights arrive as fp16 (see softmax), and one more
    // product with the reciprocals of the V scale mantissas (lds_rs) gives
    // the row sums of the values the codes times 2^e are taken with; safe
    // mode, the weights times the whole V scales as a bf16 pair (exact to
    // 2^-17), bf16 codes.
    auto weighted_values = [&](const char *vl, const float *vsc, const _Float16 *rs, const Weights &Pin_hi,
                               const Weights &Pin_lo, auto safe, auto full) __attribute__((always_inline)) {
        constexpr bool kOneF16 = kF16 || (KV == kInt8 && !decltype(safe)::value);
        Weights Phi, Plo;
        if constexpr (KV == kInt8 && !kOneF16) {
            // the weights times their tokens' V scales (token order e -> 16 (e/4) + 4 (l/16) + e%4)
            const f32x4_t vs0 = *(const f32x4_t *)(vsc + 4 * hgrp);
            const f32x4_t vs1 = *(const f32x4_t *)(vsc + 16 + 4 * hgrp);
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                const f32x4_t w0 = __builtin_bit_cast(f32x4_t, Pin_hi[cb]) * vs0;
                const f32x4_t w1 = __builtin_bit_cast(f32x4_t, Pin_lo[cb]) * vs1;
                const float pr[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
                split_weights(pr, Phi[cb], Plo[cb]);
            }
        } else {
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                Phi[cb] = Pin_hi[cb];
                Plo[cb] = Pin_lo[cb];
            }
        }
        // int8, outside the unmasked middle tiles: the lane's transpose-read
        // offsets from an opaque lane id, so the middle tiles' copies are not
        // kept past their loop
        int ln = (int)threadIdx.x;
        if constexpr (KV == kInt8 && !decltype(full)::value) __asm__ volatile("" : "+v"(ln));
        const int xl16 = ln & 15, xh = (ln >> 4) & 3;
        const int xtok = 4 * xh + (xl16 >> 2);
        const int xlane = xtok * TL::kRowBytes + 8 * (xl16 & 1);
#pragma unroll
        for (int j = 0; j < kDpl; ++j) {
            const int chunk = 2 * j + ((xl16 >> 1) & 1);
            const char *a0 = vl + xlane + ((chunk ^ TL::v_swz(xtok)) * 16);
            const i16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(a0));
            const i16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(a0 + 16 * TL::kRowBytes));
            const bf16x8_t vop = __builtin_bit_cast(
                bf16x8_t, u32x4_t{__builtin_bit_cast(u32x2_t, x0).x, __builtin_bit_cast(u32x2_t, x0).y,
                                  __builtin_bit_cast(u32x2_t, x1).x, __builtin_bit_cast(u32x2_t, x1).y});
            if constexpr (kOneF16) {
#pragma unroll
                for (int cb = 0; cb < kNc; ++cb)
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(f16x8_t, vop), __builtin_bit_cast(f16x8_t, Phi[cb]), acc[j][cb], 0, 0, 0);
                if constexpr (KV == kInt8) {
                    if (j == kDpl - 1) {
                        // row l16 of the A operand, k-elements of lane group hgrp
                        const f16x8_t rop = *(const f16x8_t *)(rs + (xl16 * 4 + xh) * 8);
#pragma unroll
                        for (int cb = 0; cb < kNc; ++cb)
                            acc_rs[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                rop, __builtin_bit_cast(f16x8_t, Phi[cb]), acc_rs[cb], 0, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int cb = 0; cb < kNc; ++cb)
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, Phi[cb], acc[j][cb], 0, 0, 0);
#pragma unroll
                for (int cb = 0; cb < kNc; ++cb)
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, Plo[cb], acc[j][cb], 0, 0, 0);
            }
        }
    };

    // The weighted sum of tile t (its V landed at least one barrier ago).
    auto pv = [&](const int t, const Weights &Ph, const Weights &Pl, auto safe, auto full) __attribute__((always_inline)) {
        if constexpr (kVt)
            weighted_values_vt(lds_v[t % kRing], Ph, safe);
        else
            weighted_values(lds_v[t % kRing], lds_vs[KV == kInt8 ? t % kVsRing : 0], &lds_rs[KV == kInt8 ? t % kRing : 0][0][0][0],
                            Ph, Pl, safe, full);
    };

    // ---- one pass over the workgroup's tiles, from a clean state.  `safe`
    // (bf16 caches only): V^T as bf16, for a workgroup whose fp16 pass met a
    // value beyond fp16.
    auto run = [&](auto safe) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kDpl; ++j)
#pragma unroll
        for (int cb = 0; cb < kNc; ++cb) acc[j][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < kNc; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.f;
        acc_rs[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    wbase = tok0 >> bs_log2;
    win = load_window(wbase);
    win_next = load_window(wbase + 64);

    // ---- prologue: the tiles the first segment reads in LDS (K(0) ..
    // K(kGroup), V(0) .. V(kGroup-2)), then the scores of tile 0.
    if constexpr (KV == kBf16) {
#pragma unroll
        for (int j = 0; j < kPiecesPerWave; ++j) {
            if (!piece_ok(j)) continue;
#pragma unroll
            for (int t = 0; t <= kGroup; ++t)
                if (t < n_tiles) issue(t, j, phys_of(t, j));
        }
#pragma nounroll
        for (int t = 0; t <= kGroup - 2; ++t) {
            if (v_stager && t < n_tiles) {
                vstage_issue(t);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                vstage_store(t, safe);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    } else {
        for (int t = 0; t < min(kGroup + 1, n_tiles); ++t) {
#pragma unroll
            for (int jj = 0; jj < kQLoads; ++jj) {
                if (!qload_ok(jj) || qload_is_v(jj)) continue;
                qissue_tile(t, jj, 0, safe);
                qstore(jj, 0, t, 0, safe);
            }
        }
        for (int t = 0; t < min(kGroup - 1, n_tiles); ++t) {
#pragma unroll
            for (int jj = 0; jj < kQLoads; ++jj) {
                if (!qload_ok(jj) || !qload_is_v(jj)) continue;
                qissue_tile(t, jj, 0, safe);
                qstore(jj, 0, 0, t, safe);
            }
        }
        // in flight into the first segment: K(kGroup+1+g) and V(kGroup-1+g)
#pragma unroll
        for (int g = 0; g < kSets; ++g)
#pragma unroll
            for (int jj = 0; jj < kQLoads; ++jj)
                if (qload_ok(jj)) qissue_tile(qload_is_v(jj) ? kGroup - 1 + g : kGroup + 1 + g, jj, g, safe);
    }
    __syncthreads();
    Scores S;                  // scores of the tile whose softmax is next
    Weights Phi, Plo;          // weights of the tile whose weighted sum is next
    if (wave_live) scores(lds_k[0], lds_sc[0][0], S, safe);
    __syncthreads();           // K(0) read by every wave before iteration 0 loads over it

    // ---- iteration i (K(i+1) and V(i-1) in LDS; the tiles of the next
    // segment loading):
    //   softmax(i)  -- vector unit, on the scores from the last iteration
    //   PV(i-1), scores(i+1)  -- matrix cores, issued among the softmax's
    //   instructions by the scheduler (independent registers)
    //   then the rescale of the accumulators if a row's max moved.
    // The first and last tiles of a wave take a general path with the
    // missing parts switched off.
    // One iteration's compute: from (Sc, Ph, Pl) -- the scores of tile i and
    // the weights of tile i-1 -- to (Sn, Pn_hi, Pn_lo).  `full`: every part
    // present (a middle tile), one straight-line block in which the compiler
    // interleaves the three independent streams.
    bool pend_grow = false;    // a softmax moved a running max: rescale before the next weighted sum
    float pend_alpha[kNc];
    auto step = [&](const int i, const Scores &Sc, const Weights &Ph, const Weights &Pl, Scores &Sn,
                    Weights &Pn_hi, Weights &Pn_lo, auto masked, auto full) __attribute__((always_inline)) {
        constexpr bool kFull = decltype(full)::value;
        const bool do_sm = kFull || i < my_steps;
        const bool do_pv = kFull || (i >= 1 && i - 1 < my_steps);
        const bool do_qk = kFull || i + 1 < my_steps;
        // the rescale the last softmax asked for: after the weighted sum of
        // tile i-2 (last iteration), before that of tile i-1
        if (pend_grow) rescale(pend_alpha, safe);
        pend_grow = false;
        if (do_sm) pend_grow = softmax(i, Sc, Pn_hi, Pn_lo, pend_alpha, masked, safe);
        if (do_pv) pv(i - 1, Ph, Pl, safe, full);
        if (do_qk) scores(lds_k[(i + 1) % kRing], lds_sc[0][(i + 1) % kRing], Sn, safe);
        // The weights are only read by the next step's weighted sum; left
        // alone, the compiler sinks their computation into that step, so one
        // block of a pair holds two softmaxes and the other bare matrix
        // products.  An empty use here keeps each softmax in its own step,
        // among the products it can be issued beside.
        if (kFull && do_sm) {
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                __asm__ volatile("" ::"v"(__builtin_bit_cast(u32x4_t, Pn_hi[cb])));
                if constexpr (!kF16 && decltype(safe)::value) __asm__ volatile("" ::"v"(__builtin_bit_cast(u32x4_t, Pn_lo[cb])));
            }
        }
    };
    auto loads = [&](const int i) __attribute__((always_inline)) {
        // The oldest block iteration i loads is V(i+kGroup-1)'s first (int8 /
        // FP8: V(i+kGroup)'s, issued at the segment's end); once it leaves the
        // window, slide.  The newest, K(i+kGroup+1)'s last (int8 / FP8:
        // K(i+2 kGroup+1)'s), is under 64 blocks further (static_assert
        // below), so a slide never skips a window.
        static_assert((KV == kBf16 ? 2 : kGroup + 1) * kTileTokens + kTileTokens - 1 < 64 * 16,
                      "a segment's loads span under 64 blocks of 16 tokens");
        if (((tok0 + (i + (KV == kBf16 ? kGroup - 1 : kGroup)) * kTileTokens) >> bs_log2) >= wbase + 64) {
            wbase += 64;
            win = win_next;
            win_next = load_window(wbase + 64);
        }
        if constexpr (KV == kBf16) {
            if (v_stager && i + kGroup - 1 < n_tiles) vstage_issue(i + kGroup - 1);
#pragma unroll
            for (int j = 0; j < kPiecesPerWave; ++j) {
                if (!piece_ok(j)) continue;
                const int tile = i + kGroup + 1;
                if (tile < n_tiles) issue(tile, j, phys_of(tile, j));
            }
        }
        return i;
    };
    // End of iteration i.  bf16: V(i+1), loaded by the staging waves during
    // this iteration, goes into its slot (no wave reads that slot in this
    // segment: its last reader, the weighted sum of V(i+1-kRing), ran in the
    // last one); at the end of a segment (`sync`: i is the segment's last
    // iteration or the workgroup's last) this wave's loads have landed, then
    // the barrier.  int8 / FP8, at the end of a segment (base its first
    // iteration): K(base+kGroup+1+g) and V(base+kGroup-1+g), loaded since the
    // last segment's end, are written to LDS (as above) -- into slots no wave
    // reads in this segment -- then K(base+2 kGroup+1+g), V(base+2 kGroup-1+g)
    // issued into the same registers, then the barrier.  The last segment may
    // be short: its stores are still those the last segment's end issued.
    auto tile_done = [&](const int i, auto more, const bool sync) __attribute__((always_inline)) {
        if constexpr (KV == kBf16) {
            if (v_stager && i + kGroup - 1 < n_tiles) {
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                vstage_store((i + kGroup - 1) % kRing, safe);
            }
            if (!sync) return;
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        } else {
            if (!sync) return;
            // base: the segment's first iteration; the registers hold what the
            // last segment's end issued
            const int base = i - i % kGroup;
#pragma unroll
            for (int g = 0; g < kSets; ++g)
#pragma unroll
                for (int jj = 0; jj < kQLoads; ++jj)
                    if (qload_ok(jj)) qstore(jj, g, base + kGroup + 1 + g, base + kGroup - 1 + g, safe);
            if (decltype(more)::value || i + 1 < n_tiles) {
#pragma unroll
                for (int g = 0; g < kSets; ++g)
#pragma unroll
                    for (int jj = 0; jj < kQLoads; ++jj)
                        if (qload_ok(jj))
                            qissue_tile(qload_is_v(jj) ? base + 2 * kGroup - 1 + g : base + 2 * kGroup + 1 + g, jj, g, safe);
            }
        }
        __syncthreads();
    };
    // Three loops, n_tiles iterations in all: the wave's first tiles (the
    // first segment), its middle tiles (every part present, no mask: one
    // straight-line body), and the rest (diagonal tiles, the last weighted
    // sum, then loads only).
    // tiles (counted from t_lo) below every row's position: no mask
    const int first_masked = (pmin >= kTileTokens - 1 ? (pmin - (kTileTokens - 1)) / kTileTokens + 1 : 0) - t_lo;
    const int full_end = wave_live ? max(1, min(first_masked, my_steps - 1)) : 1;
    Scores S2;
    Weights Phi2, Plo2;
    // a general iteration, its state copied back into (S2, P2)
    auto general = [&](const int i) __attribute__((always_inline)) {
        const int nl = loads(i);
        if (wave_live && i <= my_steps) {
            Scores Sn;
            Weights Pn_hi, Pn_lo;
            step(i, S2, Phi2, Plo2, Sn, Pn_hi, Pn_lo, std::true_type{}, std::false_type{});
#pragma unroll
            for (int cb = 0; cb < kNc; ++cb) {
                Phi2[cb] = Pn_hi[cb];
                Plo2[cb] = Pn_lo[cb];
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) S2[bb][cb] = Sn[bb][cb];
            }
        }
        tile_done(nl, std::false_type{}, i % kGroup == kGroup - 1 || i == n_tiles - 1);
    };
    int nl = loads(0);
    if (wave_live) step(0, S, Phi, Plo, S2, Phi2, Plo2, std::true_type{}, std::false_type{});
    tile_done(nl, std::false_type{}, kGroup == 1 || n_tiles == 1);
    int i = 1;
#pragma nounroll
    for (; i < kGroup && i < n_tiles; ++i) general(i);
    // The state alternates between the two register sets, so the middle
    // tiles run in pairs without copies (a pair starts a segment); after
    // the pairs it is in (S2, P2).
    for (; i + 1 < full_end; i += 2) {
        nl = loads(i);
        step(i, S2, Phi2, Plo2, S, Phi, Plo, std::false_type{}, std::true_type{});
        tile_done(nl, std::true_type{}, i % kGroup == kGroup - 1);       // i + 2 < full_end < n_tiles
        nl = loads(i + 1);
        step(i + 1, S, Phi, Plo, S2, Phi2, Plo2, std::false_type{}, std::true_type{});
        tile_done(nl, std::true_type{}, (i + 1) % kGroup == kGroup - 1);
    }
    // the general iterations (an odd middle tile, the diagonal tiles, the
    // last weighted sum, then loads only)
#pragma nounroll
    for (; i < n_tiles; ++i) general(i);
    // the last tile's weighted sum (V(n_tiles-1) landed in the last iteration)
    if (wave_live && my_steps == n_tiles) {
        if (pend_grow) rescale(pend_alpha, safe);
        pv(n_tiles - 1, Phi2, Plo2, safe, std::false_type{});
    }
    };

    // int8: the fast mode needs c within 2^-100 .. 2^100; else the safe mode runs alone
    bool rs_product = false;      // int8: the row sums are in acc_rs
    if constexpr (KV == kInt8) {
        bool again = true;
        if (i8_fast_ok) {
            run(std::false_type{});
            // every flag write of the pass came before its last barrier
            int wide = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) wide |= lds_wide[w];
            again = __builtin_amdgcn_readfirstlane(wide) != 0;
            if (again) __syncthreads();   // the pass's last LDS reads are done before the rerun loads over them
        }
        if (again) run(std::true_type{});
        rs_product = !again;
    } else {
        run(std::false_type{});
        if constexpr (kVt) {
            // every staging write of the pass came before its last barrier
            int wide = 0;
#pragma unroll
            for (int w = kVWave0; w < kVWave0 + kVWaves; ++w) wide |= lds_wide[w];
            if (__builtin_amdgcn_readfirstlane(wide) != 0) {
                __syncthreads();   // the pass's last LDS reads are done before the rerun loads over them
                run(std::true_type{});
            }
        }
    }

    if (!wave_live) return;
    // ---- the four lane groups hold partial sums over different tokens;
    // lane l has dims 16 j + 4 (l/16) + e of row l%16 of each column block.
    // One piece: the normalised rows go to out.  Several: this piece's
    // unnormalised sums, running max (log2 units, the weights' 2^kPBias
    // included) and row sum go to its partial rows, for the merge kernel.
    const int64_t prow0 = !kSplit || pieces == 1 ? 0
        : ((((int64_t)s * Hkv + g) * p.tiles_x + bx) * p.key_splits + piece) * kRowsPerGroup;
#pragma unroll
    for (int cb = 0; cb < kNc; ++cb) {
        float l = l_run[cb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if constexpr (KV == kInt8)
            if (rs_product) l = __shfl(__builtin_fmaf(acc_rs[cb][1], 0x1p-10f, acc_rs[cb][0]), l16);
        if (!colv[cb]) continue;
        const int r = row0 + 16 * cb + l16;
        if (kSplit && pieces > 1) {
            const int64_t pr = prow0 + (r - bx * kRowsPerGroup);
            float *dst = p.part_acc + pr * D + 4 * hgrp;
#pragma unroll
            for (int j = 0; j < kDpl; ++j) *(f32x4_t *)(dst + 16 * j) = acc[j][cb];
            if (hgrp == 0) *(f32x2_t *)(p.part_ml + 2 * pr) = f32x2_t{m_run[cb], l};
            continue;
        }
        const int i = r / G;
        const int hh = r - i * G;
        const float inv = 1.f / l;
        float *dst = p.out + ((int64_t)(q0 + i) * Hq + g * G + hh) * D + 4 * hgrp;
#pragma unroll
        for (int j = 0; j < kDpl; ++j) *(f32x4_t *)(dst + 16 * j) = acc[j][cb] * inv;
    }
}

// ---- key pieces: the merge.  Block b takes kMergeRows rows of row tile
// b / kMergeBlocksPerTile (unit order: sequence, kv head, row tile), D/4
// lanes a row, 4 dims each.  A row tile with one piece was written by the
// prefill kernel.  Out row = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,
// M = max_k m_k, taken piece by piece with a running max (a piece that saw
// none of the row's keys has m = -inf, l = 0, acc = 0); the loads of four
// pieces are issued together.
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void pa_prefill_merge_kernel(const PrefillParams p) {
    constexpr int kLanesPerRow = D / 4;
    constexpr int kMergeRows = kMergeThreads / kLanesPerRow;
    constexpr int kBlocksPerTile = kRowsPerGroup / kMergeRows;
    const int64_t unit = (int64_t)blockIdx.x / kBlocksPerTile;
    const int bx = (int)(unit % p.tiles_x);
    const int64_t pair = unit / p.tiles_x;
    const int g = (int)(pair % p.num_kv_heads);
    const int s = (int)(pair / p.num_kv_heads);
    const int G = p.group;
    const int q0 = p.q_offsets[s];
    const int nq = p.q_offsets[s + 1] - q0;
    const int R = nq * G;
    const int rl = (int)(blockIdx.x % kBlocksPerTile) * kMergeRows + (int)threadIdx.x / kLanesPerRow;
    const int r = bx * kRowsPerGroup + rl;
    if (r >= R) return;
    // the prefill kernel's piece count for this row tile: its last row's
    // position gives its tiles
    const int last = min(R, (bx + 1) * kRowsPerGroup) - 1;
    const int n_full = (p.context_lens[s] - nq + last / G) / kTileTokens + 1;
    const int pieces = max(1, min(p.key_splits, n_full));
    if (pieces == 1) return;
    const int d = 4 * ((int)threadIdx.x % kLanesPerRow);
    const int64_t pr0 = unit * p.key_splits * kRowsPerGroup + rl;   // piece k: + k * 256
    float M = -INFINITY, L = 0.f;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < pieces; k0 += 4) {
        f32x2_t ml[4];
        f32x4_t a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t pr = pr0 + (int64_t)min(k0 + u, pieces - 1) * kRowsPerGroup;
            ml[u] = *(const f32x2_t *)(p.part_ml + 2 * pr);
            a[u] = *(const f32x4_t *)(p.part_acc + pr * D + d);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (k0 + u >= pieces) break;
            const float m_new = fmaxf(M, ml[u][0]);
            if (m_new == -INFINITY) continue;            // nothing seen yet
            const float f_old = exp2f(M - m_new);         // 0 while M is -inf
            const float f_k = exp2f(ml[u][0] - m_new);
            L = L * f_old + ml[u][1] * f_k;
            o = o * f_old + a[u] * f_k;
            M = m_new;
        }
    }
    const int i = r / G;
    const int hh = r - i * G;
    *(f32x4_t *)(p.out + ((int64_t)(q0 + i) * p.num_q_heads + g * G + hh) * D + d) = o * (1.f / L);
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}
bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

constexpr int kMaxKeySplits = 64;

// Shape checks shared by every prefill entry point; *tiles receives the row
// tiles per (sequence, kv head).
int check_shape(const pa_prefill_shape *sh, int64_t *tiles) {
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
    *tiles = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
    if (rows >= ((int64_t)1 << 30) || *tiles > 0x7fffffff || sh->num_kv_heads > 65535 ||
        sh->num_seqs > 65535)
        return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Partial rows of a key-split call: 256 per (sequence, kv head, row tile, piece).
int64_t partial_rows(const pa_prefill_shape *sh, int64_t tiles, int key_splits) {
    return (int64_t)sh->num_seqs * sh->num_kv_heads * tiles * key_splits * kRowsPerGroup;
}

int64_t split_workspace_bytes(const pa_prefill_shape *sh, int64_t tiles, int key_splits) {
    return key_splits > 1 ? partial_rows(sh, tiles, key_splits) * (sh->head_dim + 2) * 4 : 0;
}

template <bool kSplit>
void launch_prefill(int kind, int head_dim, dim3 grid, dim3 block, hipStream_t st, const PrefillParams &p) {
    if (head_dim == 128) {
        if (kind == kInt8) hipLaunchKernelGGL((pa_prefill_kernel<128, kInt8, kSplit>), grid, block, 0, st, p);
        else if (kind == kFp8) hipLaunchKernelGGL((pa_prefill_kernel<128, kFp8, kSplit>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((pa_prefill_kernel<128, kBf16, kSplit>), grid, block, 0, st, p);
    } else {
        if (kind == kInt8) hipLaunchKernelGGL((pa_prefill_kernel<64, kInt8, kSplit>), grid, block, 0, st, p);
        else if (kind == kFp8) hipLaunchKernelGGL((pa_prefill_kernel<64, kFp8, kSplit>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((pa_prefill_kernel<64, kBf16, kSplit>), grid, block, 0, st, p);
    }
}

int prefill_common(int kind, const void *q, const void *k_cache, const void *v_cache,
                   const float *k_scales, const float *v_scales, const int32_t *block_tables,
                   const int32_t *context_lens, const int32_t *q_offsets, float scale, float *out,
                   const pa_prefill_shape *sh, int key_splits, void *workspace,
                   size_t workspace_bytes, void *stream) {
    int64_t tiles = 0;
    const int rc = check_shape(sh, &tiles);
    if (rc != PA_OK) return rc;
    if (key_splits < 1 || key_splits > kMaxKeySplits) return PA_ERR_SHAPE;
    const int group = sh->num_q_heads / sh->num_kv_heads;
    if (sh->num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !q_offsets || !out)
        return PA_ERR_NULL;
    if (kind == kInt8 && (!k_scales || !v_scales)) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return PA_ERR_ALIGNMENT;
    if (kind == kBf16 ? (!aligned16(k_cache) || !aligned16(v_cache))
                      : (((uintptr_t)k_cache | (uintptr_t)v_cache) & 7u) != 0)
        return PA_ERR_ALIGNMENT;
    if (kind == kInt8 && (((uintptr_t)k_scales | (uintptr_t)v_scales) & 3u) != 0) return PA_ERR_ALIGNMENT;
    const int64_t ws_need = split_workspace_bytes(sh, tiles, key_splits);
    if (key_splits > 1) {
        if (!workspace || workspace_bytes < (size_t)ws_need) return PA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PA_ERR_ALIGNMENT;
    }
    PrefillParams p;
    p.q = (const uint16_t *)q;
    p.k = k_cache;
    p.v = v_cache;
    p.k_scales = k_scales;
    p.v_scales = v_scales;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.q_offsets = q_offsets;
    p.out = out;
    p.scale_log2 = fabsf(scale) * kLog2e;
    p.q_sign = scale < 0.f ? 0x80008000u : 0u;
    p.num_q_heads = sh->num_q_heads;
    p.num_kv_heads = sh->num_kv_heads;
    p.group = group;
    p.max_blocks_per_seq = sh->max_blocks_per_seq;
    p.log2_block_size = ilog2(sh->block_size);
    p.num_seqs = sh->num_seqs;
    p.tiles_x = (int)tiles;
    p.key_splits = key_splits;
    p.part_acc = key_splits > 1 ? (float *)workspace : nullptr;
    p.part_ml = key_splits > 1 ? (float *)workspace + partial_rows(sh, tiles, key_splits) * sh->head_dim : nullptr;
    const int64_t units = (int64_t)sh->num_kv_heads * sh->num_seqs * tiles;
    const int64_t merge_blocks = units * (kRowsPerGroup / (kMergeThreads / (sh->head_dim / 4)));
    if (merge_blocks >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    const int64_t pairs = (int64_t)sh->num_kv_heads * sh->num_seqs;
    const int64_t n_wg = 8 * ((pairs + 7) / 8) * tiles * key_splits;
    if (n_wg >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)n_wg);
    const dim3 block(kThreads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (key_splits > 1) launch_prefill<true>(kind, sh->head_dim, grid, block, st, p);
    else launch_prefill<false>(kind, sh->head_dim, grid, block, st, p);
    if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
    if (key_splits > 1) {
        const dim3 mgrid((unsigned)merge_blocks);
        if (sh->head_dim == 128) hipLaunchKernelGGL((pa_prefill_merge_kernel<128>), mgrid, dim3(kMergeThreads), 0, st, p);
        else hipLaunchKernelGGL((pa_prefill_merge_kernel<64>), mgrid, dim3(kMergeThreads), 0, st, p);
        if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

}  // namespace

extern "C" int paged_attn_prefill(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *q_offsets, float scale, float *out,
                                  const pa_prefill_shape *sh, void *stream) {
    return prefill_common(kBf16, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                          q_offsets, scale, out, sh, 1, nullptr, 0, stream);
}

extern "C" int paged_attn_prefill_int8(const void *q, const int8_t *k_cache, const int8_t *v_cache,
                                       const float *k_scales, const float *v_scales,
                                       const int32_t *block_tables, const int32_t *context_lens,
                                       const int32_t *q_offsets, float scale, float *out,
                                       const pa_prefill_shape *sh, void *stream) {
    return prefill_common(kInt8, q, k_cache, v_cache, k_scales, v_scales, block_tables, context_lens,
                          q_offsets, scale, out, sh, 1, nullptr, 0, stream);
}

extern "C" int paged_attn_prefill_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                                      const int32_t *block_tables, const int32_t *context_lens,
                                      const int32_t *q_offsets, float scale, float *out,
                                      const pa_prefill_shape *sh, void *stream) {
    return prefill_common(kFp8, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                          q_offsets, scale, out, sh, 1, nullptr, 0, stream);
}

extern "C" int paged_attn_prefill_plan(const pa_prefill_shape *sh, int32_t *key_splits) {
    if (!key_splits) return PA_ERR_NULL;
    int64_t tiles = 0;
    const int rc = check_shape(sh, &tiles);
    if (rc != PA_OK) return rc;
    *key_splits = 1;
    const int64_t units = (int64_t)sh->num_seqs * sh->num_kv_heads * tiles;
    if (units == 0) return PA_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return PA_ERR_LAUNCH;
    // one prefill workgroup fills a compute unit: split the keys until the
    // units' pieces cover the compute units, keeping 4 or more tiles a piece
    const int64_t max_tiles = ((int64_t)sh->max_blocks_per_seq * sh->block_size + kTileTokens - 1) / kTileTokens;
    int64_t k = (cus + units - 1) / units;
    k = std::min<int64_t>(k, std::max<int64_t>(1, max_tiles / 4));
    *key_splits = (int32_t)std::max<int64_t>(1, std::min<int64_t>(k, kMaxKeySplits));
    return PA_OK;
}

extern "C" size_t paged_attn_prefill_workspace_bytes(const pa_prefill_shape *sh, int32_t key_splits) {
    int64_t tiles = 0;
    if (check_shape(sh, &tiles) != PA_OK || key_splits < 1 || key_splits > kMaxKeySplits) return 0;
    return (size_t)split_workspace_bytes(sh, tiles, key_splits);
}

extern "C" int paged_attn_prefill_split(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const int32_t *q_offsets, float scale, float *out,
                                        const pa_prefill_shape *sh, int32_t key_splits, void *workspace,
                                        size_t workspace_bytes, void *stream) {
    return prefill_common(kBf16, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                          q_offsets, scale, out, sh, key_splits, workspace, workspace_bytes, stream);
}

extern "C" int paged_attn_prefill_split_int8(const void *q, const int8_t *k_cache, const int8_t *v_cache,
                                             const float *k_scales, const float *v_scales,
                                             const int32_t *block_tables, const int32_t *context_lens,
                                             const int32_t *q_offsets, float scale, float *out,
                                             const pa_prefill_shape *sh, int32_t key_splits,
                                             void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_common(kInt8, q, k_cache, v_cache, k_scales, v_scales, block_tables, context_lens,
                          q_offsets, scale, out, sh, key_splits, workspace, workspace_bytes, stream);
}

extern "C" int paged_attn_prefill_split_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                                            const int32_t *block_tables, const int32_t *context_lens,
                                            const int32_t *q_offsets, float scale, float *out,
                                            const pa_prefill_shape *sh, int32_t key_splits,
                                            void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_common(kFp8, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens,
                          q_offsets, scale, out, sh, key_splits, workspace, workspace_bytes, stream);
}
