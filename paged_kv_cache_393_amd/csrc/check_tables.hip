// check_tables.hip -- device-side check of the caller contract of the paged
// entry points (include/paged_attn.h, paged_attn_check_tables): every context
// length lies in [0, max_blocks_per_seq * block_size], and every block-table
// entry a context uses names a block of the pool (the addressing of the
// ybb.press page "LLM 推理 KV Cache 内存管理深度工程实践", section 2.2: logical
// block t / block_size of sequence s lives in physical block
// block_tables[s][t / block_size]).
//
// The check reads only the tables and the lengths, never the cache, so it is
// safe to run on arguments that would make the other kernels read out of
// bounds.  One workgroup does it all: it starts its counters itself, needs no
// initialised memory and no atomics outside LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paged_attn.h"

namespace {

constexpr int kThreads = 1024;

struct CheckParams {
    const int32_t *block_tables;
    const int32_t *context_lens;
    int32_t *result;
    int num_seqs;
    int max_blocks_per_seq;
    int block_size;
    int num_blocks;
};

__global__ __launch_bounds__(kThreads) void check_tables_kernel(CheckParams p) {
    __shared__ int bad_count;
    __shared__ int first_bad;
    if (threadIdx.x == 0) {
        bad_count = 0;
        first_bad = 0x7fffffff;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t max_ctx = (int64_t)p.max_blocks_per_seq * p.block_size;
    // a wave per sequence, its lanes over the sequence's table entries
    for (int s = wave; s < p.num_seqs; s += kThreads / 64) {
        const int n = p.context_lens[s];
        bool bad = n < 0 || (int64_t)n > max_ctx;
        if (!bad) {
            const int nblk = (int)(((int64_t)n + p.block_size - 1) / p.block_size);
            const int32_t *row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
            bool lane_bad = false;
            for (int j = lane; j < nblk; j += 64) {
                const int32_t b = row[j];
                lane_bad |= b < 0 || b >= p.num_blocks;
            }
            bad = __ballot(lane_bad) != 0ull;
        }
        if (bad && lane == 0) {
            atomicAdd(&bad_count, 1);
            atomicMin(&first_bad, s);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        p.result[0] = bad_count;
        p.result[1] = bad_count ? first_bad : -1;
    }
}

}  // namespace

extern "C" int paged_attn_check_tables(const int32_t *block_tables, const int32_t *context_lens,
                                       int32_t num_seqs, int32_t max_blocks_per_seq,
                                       int32_t block_size, int32_t num_blocks, int32_t *result,
                                       void *stream) {
    if (num_seqs < 0 || max_blocks_per_seq < 1 || block_size < 1 || num_blocks < 1) return PA_ERR_SHAPE;
    if (!result) return PA_ERR_NULL;
    if (num_seqs > 0 && (!block_tables || !context_lens)) return PA_ERR_NULL;
    CheckParams p;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.result = result;
    p.num_seqs = num_seqs;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.block_size = block_size;
    p.num_blocks = num_blocks;
    hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
