// hash.hip -- retrieval steps 1-3 on gfx950: vocabulary projection, suffix
// n-gram formation and multi-head hashing into prime-sized tables
// ([club] 1.(1) 基于 N-gram 的稀疏哈希检索; [csdn] Engram 到底怎么工作的, first
// and second steps).  Retrieval depends only on the token sequence ([rep]
// 系统效率与扩展性), so this kernel reads nothing but tokens and the map.
//
// One wavefront covers 64 consecutive positions of one sequence.  Every lane
// compresses its own token; the older ids of its suffix n-grams come from the
// neighbouring lanes by cross-lane shuffles, and lanes 0 and 1 fetch the two
// ids just before the wave's first position (earlier tokens, the carried
// context, or PAD at a sequence start).
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ int32_t compress(int32_t x, const int32_t *__restrict__ comp_map,
                                            int32_t vocab, int32_t pad) {
    return compress_id(x, comp_map, vocab, pad);
}

__global__ __launch_bounds__(kWave *kWavesPerBlock) void hash_kernel(
    HashConsts hc, const int32_t *__restrict__ tokens, int32_t batch, int32_t seqlen,
    const int32_t *__restrict__ comp_map, const int32_t *__restrict__ prev_ctx,
    uint32_t *__restrict__ idx, uint32_t *__restrict__ bad) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t waves_per_seq = (seqlen + kWave - 1) / kWave;
    const int64_t b = wave / waves_per_seq;
    if (b >= batch) return;  // whole wave exits together
    const int32_t t0 = (int32_t)(wave - b * waves_per_seq) * kWave;
    const int32_t t = t0 + lane;
    const bool live = t < seqlen;
    const int32_t pad = hc.vocab_comp;
    const int32_t *seq = tokens + b * (int64_t)seqlen;

    int32_t raw = live ? seq[t] : 0;
    bool is_bad = live && (raw < 0 || raw >= hc.vocab);
    int32_t c = live ? compress(raw, comp_map, hc.vocab, pad) : pad;

    // ids at positions t0-2 and t0-1, held by lanes 0 and 1
    int32_t halo = pad;
    if (lane < 2) {
        int32_t p = t0 - 2 + lane;
        if (p >= 0) halo = compress(seq[p], comp_map, hc.vocab, pad);
        else if (prev_ctx) halo = prev_ctx[b * 2 + (2 + p)];
    }
    int32_t c1 = __shfl(c, (lane + kWave - 1) & (kWave - 1));  // id at t-1
    int32_t c2 = __shfl(c, (lane + kWave - 2) & (kWave - 1));  // id at t-2
    int32_t h1 = __shfl(halo, 1);              // id at t0-1
    int32_t h0 = __shfl(halo, 0);              // id at t0-2
    if (lane == 0) { c1 = h1; c2 = h0; }
    if (lane == 1) { c2 = h1; }

    uint64_t bad_mask = __ballot(is_bad);
    if (bad && lane == 0 && bad_mask) atomicAdd(bad, (uint32_t)__popcll(bad_mask));
    if (!live) return;

    const uint64_t base = (uint64_t)hc.vocab_comp + 1u;
    const uint64_t key2 = (uint64_t)c1 * base + (uint64_t)c;
    const uint64_t key3 = ((uint64_t)c2 * base + (uint64_t)c1) * base + (uint64_t)c;
    uint32_t *dst = idx + ((int64_t)b * seqlen + t) * hc.n_tables;
    const int nt = hc.n_tables;
    if ((nt & 3) == 0) {
        for (int tau = 0; tau < nt; tau += 4) {
            uint32_t r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint64_t key = hc.order_of[tau + j] == 2 ? key2 : key3;
                r[j] = mod_prime(mix64(key ^ hc.seed[tau + j]), hc.rows[tau + j], hc.magic[tau + j]);
            }
            *reinterpret_cast<u32x4_t *>(dst + tau) = u32x4_t{r[0], r[1], r[2], r[3]};
        }
    } else {
        for (int tau = 0; tau < nt; ++tau) {
            const uint64_t key = hc.order_of[tau] == 2 ? key2 : key3;
            dst[tau] = mod_prime(mix64(key ^ hc.seed[tau]), hc.rows[tau], hc.magic[tau]);
        }
    }
}

}  // namespace

void launch_hash(const HashConsts &hc, const int32_t *tokens, int32_t batch, int32_t seqlen,
                 const int32_t *comp_map, const int32_t *prev_ctx, uint32_t *idx, uint32_t *bad,
                 hipStream_t s) {
    const int64_t waves = (int64_t)batch * ((seqlen + kWave - 1) / kWave);
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    launch_kernel(hash_kernel, dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock), s, hc,
                       tokens, batch, seqlen, comp_map, prev_ctx, idx, bad);
}


}  // namespace engram
