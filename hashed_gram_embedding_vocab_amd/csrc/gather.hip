// gather.hip -- retrieval step 4 on gfx950: copy the slot rows of every table
// into the concatenated embedding E ([club] 1.(1): the heads' lookups are
// concatenated).  A pure random-row copy: HBM-bandwidth bound.
//
// Work is split into 16-byte chunks, flattened over (token, table, chunk of
// the row).  A row of d_e bf16 values is d_e/8 consecutive chunks, so the
// lanes reading one row form one contiguous (up to 160-byte) burst and the
// wave's stores to E are fully contiguous.  Each thread keeps kUnroll chunks
// in flight (indices first, then all row loads, then all stores) so enough
// random reads are outstanding to cover HBM latency.  Zipf-hot rows are
// re-served by L2 and the Infinity Cache without any explicit reuse logic.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ uint64_t div_magic(uint64_t n, uint64_t magic, int32_t d) {
    // floor(n / d) for n < 2^40 with magic = floor(2^64 / d) + 1; d == 1 -> n
    return d == 1 ? n : __umul64hi(n, magic);
}

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherConsts gc,
                                                          const uint32_t *__restrict__ idx,
                                                          int64_t total_chunks, u32x4_t *__restrict__ emb) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    uint32_t row[kUnroll];
    int32_t tau[kUnroll], ch[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = base + u * kThreads;
        const int64_t cc = c < total_chunks ? c : total_chunks - 1;
        const uint64_t tok = div_magic((uint64_t)cc, gc.magic_tok, gc.tok_chunks);
        const int32_t rem = (int32_t)(cc - (int64_t)tok * gc.tok_chunks);
        const int32_t t = (int32_t)div_magic((uint64_t)rem, gc.magic_row, gc.row_chunks);
        tau[u] = t;
        ch[u] = rem - t * gc.row_chunks;
        row[u] = __ldg(idx + tok * gc.n_tables + t);
    }
    u32x4_t val[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t r = min(row[u], gc.last_row[tau[u]]);
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(gc.table[tau[u]]) +
                           (int64_t)r * gc.row_chunks + ch[u];
        val[u] = *src;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = base + u * kThreads;
        if (c < total_chunks) emb[c] = val[u];
    }
}

}  // namespace

void launch_gather(const GatherConsts &gc, const uint32_t *idx, int64_t n_tok, void *emb,
                   hipStream_t s) {
    const int64_t total = n_tok * gc.tok_chunks;
    const int64_t per_block = (int64_t)kThreads * kUnroll;
    const int64_t blocks = (total + per_block - 1) / per_block;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, gc, idx, total,
                       reinterpret_cast<u32x4_t *>(emb));
}

}  // namespace engram
