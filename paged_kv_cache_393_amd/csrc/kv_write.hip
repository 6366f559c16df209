// kv_write.hip -- the KV write path for gfx950 (CDNA4) behind the C-ABI of
// include/paged_kv_write.h: the new tokens' key and value rows are stored at
// the token slots the block tables handed out (ybb.press page "LLM 推理 KV
// Cache 内存管理深度工程实践", section 2.1: slot = block * block_size +
// offset), optionally quantized to int8 or cast to FP8 E4M3 on the way in
// (same page, 6.1).
//
// The work is pure data movement (plus, for int8, a per-row max and a
// division per element), so the kernel is shaped for HBM: one group of
// head_dim/8 lanes owns one (token, kv head) row and moves it with one 16-byte
// load and one store per lane for K and the same for V.  The rows of one token
// are adjacent in the input and, since the cache is [blocks, block_size, kv
// heads, head_dim], also adjacent at the destination (row slot * Hkv + g), so
// every wave reads and writes whole 64..256-byte runs.
//
// int8: the row's |x| maximum is reduced across the lane group with DPP lane
// moves; scale = max / 127 (IEEE fp32 division) and code = x / scale
// rounded half to even (v_rndne_f32), clamped to [-127, 127] -- the page's
// tensor recipe in fp32.  The quotient is formed by a reciprocal multiply
// where that provably rounds to the same code, by the IEEE division elsewhere
// (see quantize8), so codes and scales are exactly those of the recipe.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_kv_write.h"

namespace {

constexpr int kThreads = 256;

struct WriteParams {
    const uint16_t *key;
    const uint16_t *value;
    const int32_t *slots;
    void *k_cache;
    void *v_cache;
    float *k_scales;
    float *v_scales;
    int64_t key_stride;    // elements
    int64_t value_stride;  // elements
    int64_t n_slots;       // num_blocks * block_size
    uint32_t rows;         // num_tokens * num_kv_heads
    uint32_t hkv;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// A DPP lane move inside each 16-lane row (kCtrl: a gfx9 dpp_ctrl value).
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Maximum over each aligned group of L lanes (8 or 16), left in every lane
// of the group, without LDS: quad permutations xor 1 and xor 2 give the max of
// each quad, the half-row mirror (lane i <-> 7 - i) joins the two quads of an
// 8-lane half, the row mirror (lane i <-> 15 - i) the two halves of a row.
// Every move reads a lane of the same group.
template <int L>
__device__ __forceinline__ float group_max(float v) {
    static_assert(L == 8 || L == 16, "groups of 8 or 16 lanes");
    v = fmaxf(v, dpp_move<0xB1>(v));     // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_move<0x4E>(v));     // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_move<0x141>(v));    // row_half_mirror
    if constexpr (L == 16) v = fmaxf(v, dpp_move<0x140>(v));   // row_mirror
    return v;
}

// Quantizes one lane's 8 values of a row whose lanes form a group of L
// (consecutive lanes); returns the 8 codes packed little-endian and the row's
// scale (the same in every lane of the group).
//
// code = rint(x / s) needs only the integer the quotient rounds to.  With
// r = rcp(s) (v_rcp_f32, within 1 ulp) the product x * r is within
// 127 * 3 * 2^-24 < 2^-15 of the correctly rounded quotient (|x| <= amax, so
// |x / s| <= 127 * (1 + 2^-23)).  Unless the product lies within 2^-12 of a
// half-integer, both round to the same integer.  Lanes where it does (about
// 1e-4 of the values) and rows whose scale is too small for a finite
// reciprocal take the IEEE division instead, so every code is exactly
// rint(x / s).
template <int L>
__device__ __forceinline__ uint2 quantize8(const uint4 w, float &scale_out) {
    float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                  bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = group_max<L>(amax);
    const float s = amax / 127.0f;
    const bool fast_row = amax >= 0x1p-96f;
    const float r = __builtin_amdgcn_rcpf(s);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float q = x[i] * r;
        const float frac = q - floorf(q);
        if (!fast_row || fabsf(frac - 0.5f) < 0x1p-12f) q = x[i] / s;
        float c = 0.0f;
        if (s != 0.0f) c = fminf(fmaxf(__builtin_rintf(q), -127.0f), 127.0f);
        const uint32_t byte = (uint32_t)(int32_t)c & 0xffu;
        packed[i / 4] |= byte << (8 * (i % 4));
    }
    scale_out = s;
    return make_uint2(packed[0], packed[1]);
}

// Casts one lane's 8 bf16 values to FP8 E4M3 codes (packed little-endian).
// v_cvt_pk_fp8_f32 rounds to nearest even, keeps subnormals and turns
// magnitudes past 464 into the NaN code with the value's sign -- the cast of
// torch's float8_e4m3fn -- except that it gives 0xFF for every NaN input; a
// NaN is therefore first replaced by the infinity of its sign, which converts
// to the NaN code of that sign.
__device__ __forceinline__ float nan_to_signed_inf(float x) {
    return __builtin_isnan(x) ? __builtin_copysignf(__builtin_inff(), x) : x;
}

__device__ __forceinline__ uint2 cast_fp8x8(const uint4 w) {
    float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                  bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = nan_to_signed_inf(x[i]);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// Element kinds of the cache written.
enum WriteKind : int { kWriteBf16 = 0, kWriteInt8 = 1, kWriteFp8 = 2 };

template <int D, int KIND>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(WriteParams p) {
    constexpr int L = D / 8;                    // lanes per row, 8 bf16 (16 B) each
    constexpr int kRowsPerGroup = kThreads / L;
    const int lane = threadIdx.x % L;
    const uint32_t row = blockIdx.x * (uint32_t)kRowsPerGroup + threadIdx.x / L;
    // Every lane of a row's group takes the same exits, so the lane moves in
    // quantize8 only ever involve lanes that are all active.
    if (row >= p.rows) return;
    const uint32_t t = row / p.hkv;
    const uint32_t g = row - t * p.hkv;
    const int32_t slot = p.slots[t];
    const uint4 kw = *reinterpret_cast<const uint4 *>(p.key + (int64_t)t * p.key_stride +
                                                      g * D + lane * 8);
    const uint4 vw = *reinterpret_cast<const uint4 *>(p.value + (int64_t)t * p.value_stride +
                                                      g * D + lane * 8);
    // int8 / fp8: the row loads are issued with the slot load, not after the
    // slot test (the empty asm keeps the compiler from sinking them below
    // it), so the conversion starts one memory round trip earlier: 26.6 ->
    // 26.0 us (int8) and 23.0 -> 22.4 us (fp8) on a 16384-token write.  The
    // plain bf16 copy measured slower that way (27 -> 34 us) and keeps the
    // loads after the test.
    if constexpr (KIND != kWriteBf16) __asm__ volatile("" ::"v"(kw.x), "v"(vw.x));
    if (slot < 0 || (int64_t)slot >= p.n_slots) return;
    const int64_t cell = (int64_t)slot * p.hkv + g;   // (block, offset, g) row of the cache
    if constexpr (KIND == kWriteBf16) {
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.k_cache) + cell * D + lane * 8) = kw;
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.v_cache) + cell * D + lane * 8) = vw;
    } else if constexpr (KIND == kWriteFp8) {
        *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(p.k_cache) + cell * D + lane * 8) = cast_fp8x8(kw);
        *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(p.v_cache) + cell * D + lane * 8) = cast_fp8x8(vw);
    } else {
        float ks, vs;
        const uint2 kc = quantize8<L>(kw, ks);
        const uint2 vc = quantize8<L>(vw, vs);
        *reinterpret_cast<uint2 *>(static_cast<int8_t *>(p.k_cache) + cell * D + lane * 8) = kc;
        *reinterpret_cast<uint2 *>(static_cast<int8_t *>(p.v_cache) + cell * D + lane * 8) = vc;
        if (lane == 0) {
            p.k_scales[cell] = ks;
            p.v_scales[cell] = vs;
        }
    }
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int write_common(const void *key, const void *value, const int32_t *slots, void *kc, void *vc,
                 float *ks, float *vs, const pa_write_shape *sh, void *stream, int kind) {
    const bool int8 = kind == kWriteInt8;
    if (!sh) return PA_ERR_NULL;
    if (sh->num_tokens < 0 || sh->num_kv_heads < 1 || sh->block_size < 1 || sh->num_blocks < 1 ||
        sh->key_stride < 0 || sh->value_stride < 0)
        return PA_ERR_SHAPE;
    if (sh->head_dim != 64 && sh->head_dim != 128) return PA_ERR_UNSUPPORTED;
    const int64_t row = (int64_t)sh->num_kv_heads * sh->head_dim;
    const int64_t kst = sh->key_stride ? sh->key_stride : row;
    const int64_t vst = sh->value_stride ? sh->value_stride : row;
    if (kst < row || vst < row) return PA_ERR_SHAPE;
    const int64_t rows = (int64_t)sh->num_tokens * sh->num_kv_heads;
    if (rows >= ((int64_t)1 << 27)) return PA_ERR_UNSUPPORTED;
    if (rows == 0) return PA_OK;   // nothing to store; the pointers are not looked at
    if (!key || !value || !slots || !kc || !vc) return PA_ERR_NULL;
    if (int8 && (!ks || !vs)) return PA_ERR_NULL;
    if (!aligned(key, 16) || !aligned(value, 16) || kst % 8 || vst % 8) return PA_ERR_ALIGNMENT;
    if (kind == kWriteBf16 ? (!aligned(kc, 16) || !aligned(vc, 16))
                           : (!aligned(kc, 8) || !aligned(vc, 8)))
        return PA_ERR_ALIGNMENT;
    if (int8 && (!aligned(ks, 4) || !aligned(vs, 4))) return PA_ERR_ALIGNMENT;

    WriteParams p;
    p.key = static_cast<const uint16_t *>(key);
    p.value = static_cast<const uint16_t *>(value);
    p.slots = slots;
    p.k_cache = kc;
    p.v_cache = vc;
    p.k_scales = ks;
    p.v_scales = vs;
    p.key_stride = kst;
    p.value_stride = vst;
    p.n_slots = (int64_t)sh->num_blocks * sh->block_size;
    p.rows = (uint32_t)rows;
    p.hkv = (uint32_t)sh->num_kv_heads;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int rows_per_group = kThreads / (sh->head_dim / 8);
    const dim3 grid((unsigned)((rows + rows_per_group - 1) / rows_per_group));
    const dim3 block(kThreads);
    if (sh->head_dim == 128) {
        if (kind == kWriteInt8) hipLaunchKernelGGL((kv_write_kernel<128, kWriteInt8>), grid, block, 0, st, p);
        else if (kind == kWriteFp8) hipLaunchKernelGGL((kv_write_kernel<128, kWriteFp8>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((kv_write_kernel<128, kWriteBf16>), grid, block, 0, st, p);
    } else {
        if (kind == kWriteInt8) hipLaunchKernelGGL((kv_write_kernel<64, kWriteInt8>), grid, block, 0, st, p);
        else if (kind == kWriteFp8) hipLaunchKernelGGL((kv_write_kernel<64, kWriteFp8>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((kv_write_kernel<64, kWriteBf16>), grid, block, 0, st, p);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int paged_kv_write(const void *key, const void *value, const int32_t *slot_mapping,
                   void *k_cache, void *v_cache, const pa_write_shape *shape, void *stream) {
    return write_common(key, value, slot_mapping, k_cache, v_cache, nullptr, nullptr, shape,
                        stream, kWriteBf16);
}

int paged_kv_write_fp8(const void *key, const void *value, const int32_t *slot_mapping,
                       uint8_t *k_cache, uint8_t *v_cache, const pa_write_shape *shape,
                       void *stream) {
    return write_common(key, value, slot_mapping, k_cache, v_cache, nullptr, nullptr, shape,
                        stream, kWriteFp8);
}

int paged_kv_write_int8(const void *key, const void *value, const int32_t *slot_mapping,
                        int8_t *k_cache, int8_t *v_cache, float *k_scales, float *v_scales,
                        const pa_write_shape *shape, void *stream) {
    return write_common(key, value, slot_mapping, k_cache, v_cache, k_scales, v_scales, shape,
                        stream, kWriteInt8);
}

}  // extern "C"
