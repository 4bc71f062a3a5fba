// offload.hip -- retrieval from tables that live in host memory, with the
// Zipf-hot rows kept in HBM.
//
// The pages' deployment keeps the tables in host DRAM and fetches the rows a
// step needs over the host link, ahead of the layer that uses them (the
// indices depend only on the tokens), with a multi-level cache because n-gram
// access is Zipfian ([rep] 工程实现与硬件效率, 技术方案; [csdn] 实际效果到底有多好).
// Here the GPU reads the rows of pinned host memory itself (no CPU copy
// thread, no staging buffer): one 16-byte load per lane, many in flight, the
// same chunk layout as the HBM gather.  Rows the caller names as hot are
// copied once into an HBM cache per table, found through an open-addressing
// hash of the row number (linear probing, load factor at most 1/2), so hot
// rows cost an HBM read instead of a host-link read.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;  // row chunks in flight per thread

// First probe slot of a row: the top bits of a Fibonacci-hashed row number
// (rows come out of a 64-bit mix already; this only spreads neighbours).
__device__ __forceinline__ uint32_t cache_slot0(uint32_t row, uint32_t capacity) {
    return (uint32_t)(((uint64_t)(row * 0x9E3779B1u) * capacity) >> 32);
}

__global__ __launch_bounds__(kThreads) void cache_clear_kernel(uint32_t *keys, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) keys[i] = 0u;
}

// One thread per (table, hot entry): claim the first free slot of the row's
// probe sequence (key = row + 1; 0 marks a free slot).  Entries naming a row
// outside the table, or a row already present, claim nothing.
__global__ __launch_bounds__(kThreads) void cache_insert_kernel(GatherConsts gc, uint32_t capacity,
                                                                const uint32_t *hot, int32_t n_hot, uint32_t *keys) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)gc.n_tables * n_hot) return;
    const int tau = (int)(i / n_hot);
    const uint32_t row = hot[i];
    if (row > gc.last_row[tau]) return;
    uint32_t *k = keys + (int64_t)tau * capacity;
    uint32_t s = cache_slot0(row, capacity);
    for (uint32_t probe = 0; probe < capacity; ++probe) {
        const uint32_t old = atomicCAS(k + s, 0u, row + 1u);
        if (old == 0u || old == row + 1u) return;
        s = s + 1u == capacity ? 0u : s + 1u;
    }
}

// One thread per 16-byte chunk of every slot: copy the claimed rows from the
// tables into the cache.
__global__ __launch_bounds__(kThreads) void cache_fill_kernel(GatherConsts gc, uint32_t capacity,
                                                              const uint32_t *keys, u32x4_t *rows) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t slot = i / gc.row_chunks;
    if (slot >= (int64_t)gc.n_tables * capacity) return;
    const int ch = (int)(i - slot * gc.row_chunks);
    const uint32_t key = keys[slot];
    if (key == 0u) return;
    const int tau = (int)(slot / capacity);
    rows[i] = reinterpret_cast<const u32x4_t *>(gc.table[tau])[(int64_t)(key - 1u) * gc.row_chunks + ch];
}

// A block handles kGroups groups of tpb = 256 / n_tables consecutive tokens
// per iteration: iteration i, i + gridDim.x, ... (one iteration per block
// unless the launch caps its workgroups).  Phase 1: one thread per (token,
// table) pair of each group reads the slot, looks it up in the table's cache
// (when there is one) and leaves the row's source address in LDS; the
// groups' lookups are independent, so they overlap.  Phase 2: the block
// copies the rows in 16-byte chunks, kUnroll loads in flight per thread (a
// capped launch keeps enough bytes in flight on few CUs to fill the host
// link), the lanes of one row reading one contiguous burst.
constexpr int kGroups = 4;
// Row addresses kept in LDS as global-address-space pointers: generic ones
// make the copies flat loads, which also count as LDS operations, so each
// LDS read of the next address would wait for the previous row.  (Pinned
// host tables are reached through the same global addresses.)
typedef const __attribute__((address_space(1))) u32x4_t *grow_t;

__global__ __launch_bounds__(kThreads) void cached_gather_kernel(GatherConsts gc, uint32_t capacity,
                                                                 const uint32_t *__restrict__ idx, int64_t n_tok,
                                                                 int32_t tpb, const uint32_t *__restrict__ keys,
                                                                 const u32x4_t *__restrict__ cache_rows,
                                                                 u32x4_t *__restrict__ emb) {
    __shared__ grow_t src_s[kGroups * kThreads];
    const int n_tables = gc.n_tables;
    const int64_t per_iter = (int64_t)tpb * kGroups;
    const int64_t n_iters = (n_tok + per_iter - 1) / per_iter;
    for (int64_t it = blockIdx.x; it < n_iters; it += gridDim.x) {
        const int64_t tok0 = it * per_iter;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const int pr = threadIdx.x;
            const int tl = pr / n_tables;
            const int tau = pr - tl * n_tables;
            const int64_t tok = tok0 + (int64_t)g * tpb + tl;
            if (tl < tpb && tok < n_tok) {
                const uint32_t row = min(idx[tok * n_tables + tau], gc.last_row[tau]);
                const u32x4_t *src =
                    reinterpret_cast<const u32x4_t *>(gc.table[tau]) + (int64_t)row * gc.row_chunks;
                if (capacity != 0u) {
                    const uint32_t *k = keys + (int64_t)tau * capacity;
                    uint32_t s = cache_slot0(row, capacity);
                    for (uint32_t probe = 0; probe < capacity; ++probe) {
                        const uint32_t key = k[s];
                        if (key == row + 1u) {
                            src = cache_rows + ((int64_t)tau * capacity + s) * gc.row_chunks;
                            break;
                        }
                        if (key == 0u) break;
                        s = s + 1u == capacity ? 0u : s + 1u;
                    }
                }
                src_s[g * kThreads + pr] = (grow_t)src;
            }
        }
        __syncthreads();
        const int64_t ntok_here = min<int64_t>(per_iter, n_tok - tok0);
        const int chunks = (int)ntok_here * gc.tok_chunks;
        u32x4_t *dst = emb + tok0 * gc.tok_chunks;
        for (int c0 = threadIdx.x; c0 < chunks; c0 += kThreads * kUnroll) {
            u32x4_t val[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = min(c0 + u * kThreads, chunks - 1);
                const int tl = c / gc.tok_chunks;  // token within the iteration
                const int rem = c - tl * gc.tok_chunks;
                const int tau = rem / gc.row_chunks;
                const int ch = rem - tau * gc.row_chunks;
                const int g = tl / tpb;
                val[u] = src_s[g * kThreads + (tl - g * tpb) * n_tables + tau][ch];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + u * kThreads;
                if (c < chunks) dst[c] = val[u];
            }
        }
        __syncthreads();  // src_s is rewritten by the next iteration
    }
}

// Host-gather prefetch: the host threads looked every (token, table) pair up
// in a copy of the cache keys; code[pair] is the cache slot of a hit, or
// kMissBit | the staged row of a miss.
constexpr uint32_t kMissBit = 0x80000000u;

// E from the cache rows (hits) and the staged rows (misses), one
// 16-byte chunk per thread, kUnroll in flight.
__global__ __launch_bounds__(kThreads) void prefetch_assemble_kernel(GatherConsts gc, int64_t total_chunks,
                                                                     const uint32_t *__restrict__ code,
                                                                     const u32x4_t *__restrict__ cache_rows,
                                                                     const u32x4_t *__restrict__ staged,
                                                                     u32x4_t *__restrict__ emb) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    u32x4_t val[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = min(base + u * kThreads, total_chunks - 1);
        const int64_t pr = c / gc.row_chunks;
        const int ch = (int)(c - pr * gc.row_chunks);
        const uint32_t k = code[pr];
        const u32x4_t *src = (k & kMissBit) ? staged + (int64_t)(k & ~kMissBit) * gc.row_chunks
                                            : cache_rows + (int64_t)k * gc.row_chunks;
        val[u] = src[ch];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = base + u * kThreads;
        if (c < total_chunks) emb[c] = val[u];
    }
}

}  // namespace

void launch_cache_build(const GatherConsts &gc, uint32_t capacity, const uint32_t *hot, int32_t n_hot,
                        uint32_t *keys, void *rows, hipStream_t s) {
    const int64_t n_keys = (int64_t)gc.n_tables * capacity;
    launch_kernel(cache_clear_kernel, dim3((unsigned)((n_keys + kThreads - 1) / kThreads)), dim3(kThreads), s, keys,
                  n_keys);
    const int64_t n_ins = (int64_t)gc.n_tables * n_hot;
    if (n_ins > 0)
        launch_kernel(cache_insert_kernel, dim3((unsigned)((n_ins + kThreads - 1) / kThreads)), dim3(kThreads), s,
                      gc, capacity, hot, n_hot, keys);
    const int64_t n_chunks = n_keys * gc.row_chunks;
    launch_kernel(cache_fill_kernel, dim3((unsigned)((n_chunks + kThreads - 1) / kThreads)), dim3(kThreads), s, gc,
                  capacity, keys, reinterpret_cast<u32x4_t *>(rows));
}

void launch_cached_gather(const GatherConsts &gc, uint32_t capacity, const uint32_t *idx, int64_t n_tok,
                          const uint32_t *keys, const void *rows, void *emb, int32_t max_workgroups,
                          hipStream_t s) {
    const int tpb = kThreads / gc.n_tables;
    const int64_t per_iter = (int64_t)tpb * kGroups;
    int64_t blocks = (n_tok + per_iter - 1) / per_iter;
    if (max_workgroups > 0 && blocks > max_workgroups) blocks = max_workgroups;
    launch_kernel(cached_gather_kernel, dim3((unsigned)blocks), dim3(kThreads), s, gc, capacity, idx, n_tok, tpb,
                  keys, reinterpret_cast<const u32x4_t *>(rows), reinterpret_cast<u32x4_t *>(emb));
}

void launch_prefetch_assemble(const GatherConsts &gc, int64_t n_tok, const uint32_t *code, const void *cache_rows,
                              const void *staged, void *emb, hipStream_t s) {
    const int64_t total = n_tok * gc.tok_chunks;
    const int64_t per_block = (int64_t)kThreads * kUnroll;
    launch_kernel(prefetch_assemble_kernel, dim3((unsigned)((total + per_block - 1) / per_block)), dim3(kThreads), s,
                  gc, total, code, reinterpret_cast<const u32x4_t *>(cache_rows),
                  reinterpret_cast<const u32x4_t *>(staged), reinterpret_cast<u32x4_t *>(emb));
}

}  // namespace engram

