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
// Row loads are nontemporal: measured on the 200 GB tables, the fused
// retrieval took 42.3 us per 32k tokens against 44.6 with ordinary loads (Zipf
// tokens) and 42.4 against 46.8 (uniform tokens); nontemporal E stores were
// slower (E is read again right away by the projections).
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;    // chunks in flight per thread (index-driven gather)
#ifndef ENGRAM_HG_UNROLL
#define ENGRAM_HG_UNROLL 10
#endif
#ifndef ENGRAM_HG_NT
#define ENGRAM_HG_NT 1
#endif
constexpr int kHGUnroll = ENGRAM_HG_UNROLL; // row chunks in flight per thread in the fused kernel
constexpr bool kNtRows = (ENGRAM_HG_NT & 1) != 0;  // nontemporal row loads
constexpr bool kNtEmb = (ENGRAM_HG_NT & 2) != 0;   // nontemporal E stores

// Table rows through global-address-space pointers: through generic ones
// the loads become flat loads, which also count as LDS operations, so the
// LDS read of the next pointer would wait for the previous row.
typedef const __attribute__((address_space(1))) u32x4_t *grow_t;
__device__ __forceinline__ u32x4_t load_row_chunk(grow_t p) {
    if constexpr (kNtRows) return __builtin_nontemporal_load(p);
    return *p;
}
__device__ __forceinline__ void store_emb_chunk(u32x4_t *p, u32x4_t v) {
    if constexpr (kNtEmb) __builtin_nontemporal_store(v, p);
    else *p = v;
}

__device__ __forceinline__ uint64_t div_magic(uint64_t n, uint64_t magic, int32_t d) {
    // floor(n / d) for n < 2^40 with magic = floor(2^64 / d) + 1; d == 1 -> n
    return d == 1 ? n : __umul64hi(n, magic);
}

// The table bases (and last rows) go to LDS first: indexed at run time, the
// kernel-argument arrays would be read from memory by a vector load in front
// of every row load, each waiting for all earlier loads, so a thread's row
// loads would go out one at a time instead of together.
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherConsts gc,
                                                          const uint32_t *__restrict__ idx,
                                                          int64_t total_chunks, u32x4_t *__restrict__ emb) {
    __shared__ grow_t tab_s[kMaxTables];
    __shared__ uint32_t last_s[kMaxTables];
    if (threadIdx.x < (unsigned)gc.n_tables) {
        tab_s[threadIdx.x] = (grow_t)(gc.table[threadIdx.x]);
        last_s[threadIdx.x] = gc.last_row[threadIdx.x];
    }
    __syncthreads();
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
        const uint32_t r = min(row[u], last_s[tau[u]]);
        const grow_t src = tab_s[tau[u]] + (int64_t)r * gc.row_chunks + ch[u];
        val[u] = load_row_chunk(src);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = base + u * kThreads;
        if (c < total_chunks) store_emb_chunk(emb + c, val[u]);
    }
}

// Fused retrieval (engram_forward): a block owns tpb = 256 / n_tables
// consecutive tokens.  Phase 1: one thread per
// (token, table) pair forms the token's suffix n-gram from the raw ids (ids
// before a sequence's first token come from prev_ctx, else PAD), hashes it
// with the table's seed and leaves the slot in LDS.  Phase 2: the block
// copies the pairs' rows in 16-byte chunks, up to kHGUnroll loads in flight
// per thread.  The slots never travel through HBM.  With one token per
// sequence, ctx_out (the same array as prev_ctx, or null) is rolled by the
// block after its barrier: every read of a sequence's context is in the block
// that owns its token.
__global__ __launch_bounds__(kThreads) void hash_gather_kernel(
    HashConsts hc, GatherConsts gc, const int32_t *__restrict__ tokens, int64_t n_tok, int32_t seqlen,
    uint64_t magic_seq, int32_t tpb, const int32_t *__restrict__ comp_map, const int32_t *prev_ctx,
    int32_t *ctx_out, uint32_t *__restrict__ bad, u32x4_t *__restrict__ emb) {
    __shared__ uint32_t slot_s[kThreads];
    __shared__ grow_t tab_s[kMaxTables];  // table bases (see gather_kernel)
    const int64_t tok0 = (int64_t)blockIdx.x * tpb;
    const int n_tables = gc.n_tables;
    if (threadIdx.x < (unsigned)n_tables) tab_s[threadIdx.x] = (grow_t)(gc.table[threadIdx.x]);
    const int pairs = tpb * n_tables;
    {
        const int pr = threadIdx.x;
        const int tl = pr / n_tables;
        const int tau = pr - tl * n_tables;
        const int64_t tok = tok0 + tl;
        if (pr < pairs && tok < n_tok) {
            const int32_t pad = hc.vocab_comp;
            const uint64_t B = (uint64_t)hc.vocab_comp + 1u;
            const int64_t b = (int64_t)div_magic((uint64_t)tok, magic_seq, seqlen);
            const int32_t t = (int32_t)(tok - b * seqlen);
            const int32_t x0 = tokens[tok];
            const int32_t c0 = compress_id(x0, comp_map, hc.vocab, pad);
            int32_t c1, c2;
            if (t >= 1) c1 = compress_id(tokens[tok - 1], comp_map, hc.vocab, pad);
            else c1 = prev_ctx ? prev_ctx[b * 2 + 1] : pad;
            if (t >= 2) c2 = compress_id(tokens[tok - 2], comp_map, hc.vocab, pad);
            else if (t == 1) c2 = prev_ctx ? prev_ctx[b * 2 + 1] : pad;
            else c2 = prev_ctx ? prev_ctx[b * 2 + 0] : pad;
            const uint64_t key = hc.order_of[tau] == 2 ? (uint64_t)c1 * B + (uint64_t)c0
                                                       : ((uint64_t)c2 * B + (uint64_t)c1) * B + (uint64_t)c0;
            slot_s[pr] = mod_prime(mix64(key ^ hc.seed[tau]), hc.rows[tau], hc.magic[tau]);
            if (bad && tau == 0 && (x0 < 0 || x0 >= hc.vocab)) atomicAdd(bad, 1u);
        }
    }
    __syncthreads();
    const int64_t ntok_here = min<int64_t>(tpb, n_tok - tok0);
    if (ctx_out && threadIdx.x < ntok_here) {  // seqlen == 1: token tok0 + i is sequence tok0 + i
        const int64_t b = tok0 + threadIdx.x;
        const int32_t n1 = compress_id(tokens[b], comp_map, hc.vocab, hc.vocab_comp);
        ctx_out[b * 2 + 0] = ctx_out[b * 2 + 1];
        ctx_out[b * 2 + 1] = n1;
    }
    const int chunks = (int)ntok_here * gc.tok_chunks;
    u32x4_t *dst = emb + tok0 * gc.tok_chunks;
    for (int c0 = threadIdx.x; c0 < chunks; c0 += kThreads * kHGUnroll) {
        u32x4_t val[kHGUnroll];
#pragma unroll
        for (int u = 0; u < kHGUnroll; ++u) {
            const int c = min(c0 + u * kThreads, chunks - 1);
            const int tl = (int)div_magic((uint64_t)c, gc.magic_tok, gc.tok_chunks);
            const int rem = c - tl * gc.tok_chunks;
            const int tau = (int)div_magic((uint64_t)rem, gc.magic_row, gc.row_chunks);
            const int ch = rem - tau * gc.row_chunks;
            const uint32_t r = slot_s[tl * n_tables + tau];
            val[u] = load_row_chunk(tab_s[tau] + (int64_t)r * gc.row_chunks + ch);
        }
#pragma unroll
        for (int u = 0; u < kHGUnroll; ++u) {
            const int c = c0 + u * kThreads;
            if (c < chunks) store_emb_chunk(dst + c, val[u]);
        }
    }
}

// The carried context after a chunk, one thread per sequence (for a
// retrieval launched on its own, after it has read the old context).
__global__ __launch_bounds__(kThreads) void ctx_kernel(CtxUpdate c, int32_t batch, int32_t seqlen) {
    const int32_t b = (int32_t)(blockIdx.x * kThreads + threadIdx.x);
    if (b < batch) ctx_update_one(c, b, seqlen);
}

}  // namespace

void launch_ctx_update(const CtxUpdate &c, int32_t batch, int32_t seqlen, hipStream_t s) {
    launch_kernel(ctx_kernel, dim3((unsigned)((batch + kThreads - 1) / kThreads)), dim3(kThreads), s, c, batch,
                  seqlen);
}

void launch_hash_gather(const HashConsts &hc, const GatherConsts &gc, const int32_t *tokens,
                        int32_t batch, int32_t seqlen, const int32_t *comp_map,
                        const int32_t *prev_ctx, uint32_t *bad, void *emb, hipStream_t s, int32_t *ctx_out) {
    const int64_t n_tok = (int64_t)batch * seqlen;
    const int tpb = kThreads / gc.n_tables;
    const int64_t blocks = (n_tok + tpb - 1) / tpb;
    const uint64_t magic_seq = seqlen <= 1 ? 0 : (uint64_t)(((unsigned __int128)1 << 64) / (unsigned)seqlen) + 1;
    launch_kernel(hash_gather_kernel, dim3((unsigned)blocks), dim3(kThreads), s, hc, gc, tokens, n_tok,
                       seqlen, magic_seq, tpb, comp_map, prev_ctx, seqlen == 1 ? ctx_out : nullptr, bad,
                       reinterpret_cast<u32x4_t *>(emb));
}

void launch_gather(const GatherConsts &gc, const uint32_t *idx, int64_t n_tok, void *emb,
                   hipStream_t s) {
    const int64_t total = n_tok * gc.tok_chunks;
    const int64_t per_block = (int64_t)kThreads * kUnroll;
    const int64_t blocks = (total + per_block - 1) / per_block;
    launch_kernel(gather_kernel, dim3((unsigned)blocks), dim3(kThreads), s, gc, idx, total,
                       reinterpret_cast<u32x4_t *>(emb));
}

}  // namespace engram
