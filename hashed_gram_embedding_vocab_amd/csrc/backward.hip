// backward.hip -- the backward of one Engram layer on gfx950, for training
// ([csdn] 实际效果到底有多好: the table slots become meaningful through the
// gradients that reach them).  The derivative of the forward of
// proj_bf16.hip / fuse.hip, for whole sequences (no carried state):
//   bwd_gate_stats_kernel  rh, rk, s and alpha of every token and branch, from
//                          the gate partials that the k/v recompute leaves
//   bwd_conv_kernel        dconv from dout, du through the transposed
//                          (anti-causal) conv, dalpha = <v, du>, dv = sum over
//                          branches of alpha du, and the conv taps' gradient
//   bwd_gate_kernel        ds = dalpha alpha (1 - alpha), then both RMSNorms
//                          backwards: dh, dk and the gammas' gradients
//   table rows             (table, row) keys sorted stably by a segmented
//                          radix sort; fixed 64-item chunks of the sorted items
//                          add the tokens' dE slices in token order
// The contractions themselves run on proj_bf16.hip's main loop: k and v
// (with the gate partials) in mode 5, dE in mode 6 (W read K-major: the
// contraction runs over its rows), dW in mode 4 (E and [dk | dv] read
// K-major: the contraction runs over tokens).  No operand is transposed.
#include <cstring>


#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kConvPos = 32;     // positions per bwd_conv_kernel workgroup
constexpr int kGateTok = 64;     // tokens per bwd_gate_kernel workgroup
constexpr int kGateGroup = 8;    // tokens whose loads bwd_gate_kernel issues together

template <typename T, int N>
__device__ __forceinline__ T pick_arg(const T (&arr)[N], int i) {
    T p = arr[0];
#pragma unroll
    for (int j = 1; j < N; ++j)
        if (i == j) p = arr[j];
    return p;
}

__device__ __forceinline__ float sigmoid_b(float x) { return 1.f / (1.f + expf(-x)); }

__device__ __forceinline__ f32x4_t load_bf16x4(const void *base, int64_t elem) {
    const u32x2_t x = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(base) + elem);
    return f32x4_t{bf16_to_f32(x[0] & 0xFFFFu), bf16_to_f32(x[0] >> 16), bf16_to_f32(x[1] & 0xFFFFu),
                   bf16_to_f32(x[1] >> 16)};
}

__device__ __forceinline__ void store_bf16x4(void *base, int64_t elem, f32x4_t v) {
    *reinterpret_cast<u32x2_t *>(reinterpret_cast<uint16_t *>(base) + elem) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Sum over the 64 lanes of a wave (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// ---------------------------------------------------------------- gate statistics
// One workgroup per (token, branch).  stats = [rh | rk | s | alpha], each [B_r][n_tok].
// One thread per (token, branch): the three sums over d (h gamma_h gamma_k k,
// k^2, h^2), added part by part in order from the k/v projection's
// per-128-channel partials, give rh, rk, s and alpha.
__global__ __launch_bounds__(256) void bwd_gate_stats_kernel(BwdArgs a) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    if (t >= a.n_tok) return;
    const float *pp = a.partials + (int64_t)m * a.n_parts * 3 * a.n_tok + t;
    float shk = 0.f, skk = 0.f, shh = 0.f;
    for (int q = 0; q < a.n_parts; ++q) {
        shk += pp[(3 * q + 0) * a.n_tok];
        skk += pp[(3 * q + 1) * a.n_tok];
        shh += pp[(3 * q + 2) * a.n_tok];
    }
    const int d = a.d;
    const float rh = sqrtf(shh / (float)d + a.eps);
    const float rk = sqrtf(skk / (float)d + a.eps);
    const float s = shk / (rh * rk) * rsqrtf((float)d);
    const int64_t plane = (int64_t)a.n_branches * a.n_tok;
    const int64_t i = (int64_t)m * a.n_tok + t;
    a.stats[i] = rh;
    a.stats[plane + i] = rk;
    a.stats[2 * plane + i] = s;
    a.stats[3 * plane + i] = sigmoid_b(s);
}

// ---------------------------------------------------------------- conv and gated value
// Workgroup (position chunk, sequence, 1024-channel stripe); each thread owns
// four channels of the chunk's positions, taken kConvSub at a time.  For the
// outputs t = s0 .. s0+kConvSub-1 of one batch, every value the batch needs
// is loaded at once (v at s0-3 .. s0+kConvSub-1, or .. s0+kConvSub+2 with
// SILU_SKIP, and every branch's dout at s0 .. s0+kConvSub+2), so a thread
// waits for memory once per batch instead of once per position; the halo
// positions shared by neighbouring batches come from the caches.  Per branch:
//   u_p = alpha_p v_p;  conv_p = sum_j w[K-1-j] u_{p-j}
//   dconv_p = dout_p (LINEAR) or dout_p (sig + conv sig (1 - sig)) (SILU_SKIP)
//   du_t = [SILU_SKIP] dout_t + sum_j w[K-1-j] dconv_{t+j}
//   dw[K-1-j] += u_{t-j} dconv_t
// Out: dv_t = sum_m alpha_t du_t (bf16, into the v columns of dkv), the
// workgroup's share of dalpha_t = <v_t, du_t> per branch, and its share of
// the taps' gradient.
constexpr int kConvSub = 4;

template <int BR, bool SILU>
__global__ __launch_bounds__(256) void bwd_conv_kernel(BwdArgs a) {
    __shared__ float alpha_s[BR][kConvPos + 6];   // positions t0-3 .. t1+2
    __shared__ float red[BR][kConvPos][4];        // per-wave dalpha shares
    constexpr int P = kConvSub;
    constexpr int NV = SILU ? P + 6 : P + 3;      // v at s0-3 .. s0-3+NV-1
    constexpr int NG = P + 3;                     // dout at s0 .. s0+P+2
    const int T = a.seqlen;
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kConvPos;
    const int t1 = min(t0 + kConvPos, T);
    const int64_t row0 = (int64_t)b * T;
    const int d = a.d;
    const int kc = a.conv_k;
    const int tid = threadIdx.x;
    const int c0 = (blockIdx.z * 256 + tid) * 4;
    const bool live = c0 < d;
    const float *alpha_all = a.stats + 3 * (int64_t)a.n_branches * a.n_tok;

    for (int x = tid; x < BR * (kConvPos + 6); x += 256) {
        const int m = x / (kConvPos + 6), j = x - m * (kConvPos + 6);
        const int p = t0 - 3 + j;
        alpha_s[m][j] = (p >= 0 && p < T) ? alpha_all[(int64_t)m * a.n_tok + row0 + p] : 0.f;
    }
    __syncthreads();

    f32x4_t wt[4];  // wt[j][c]: tap multiplying u_{t-j} (zero beyond K_c)
    f32x4_t dw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dw[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wt[j][r] = (live && j < kc) ? a.conv_w[(int64_t)(c0 + r) * kc + (kc - 1 - j)] : 0.f;
    }
    // loads read a valid address (position and channel clamped) and are
    // zeroed afterwards: no branch around them, so all of a batch's loads are
    // in flight together
    const int cc = live ? c0 : 0;
    const float *vcol = a.kv + (int64_t)a.n_branches * d + cc;
    const uint16_t *gcol = reinterpret_cast<const uint16_t *>(a.dout) + row0 * d + cc;
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    auto unpack = [](u32x2_t x) {
        return f32x4_t{bf16_to_f32(x[0] & 0xFFFFu), bf16_to_f32(x[0] >> 16), bf16_to_f32(x[1] & 0xFFFFu),
                       bf16_to_f32(x[1] >> 16)};
    };
    auto inseq = [&](int p) { return live && p >= 0 && p < T; };

    for (int s0 = t0; s0 < t1; s0 += P) {
        f32x4_t vv[NV];
        u32x2_t gg[BR][NG];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int pc = min(max(s0 - 3 + i, 0), T - 1);
            vv[i] = *reinterpret_cast<const f32x4_t *>(vcol + (row0 + pc) * a.kv_ld);
        }
#pragma unroll
        for (int m = 0; m < BR; ++m)
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int pc = min(s0 + i, T - 1);
                gg[m][i] = *reinterpret_cast<const u32x2_t *>(gcol + ((int64_t)m * a.n_tok + pc) * d);
            }
#pragma unroll
        for (int i = 0; i < NV; ++i) vv[i] = inseq(s0 - 3 + i) ? vv[i] : zero4;

        f32x4_t dv[P];
#pragma unroll
        for (int k = 0; k < P; ++k) dv[k] = zero4;
#pragma unroll
        for (int m = 0; m < BR; ++m) {
            // alpha at s0-3+i (LDS index s0-t0+i)
            float al[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) al[i] = alpha_s[m][s0 - t0 + i];
            // dconv at s0+i, zero outside the sequence
            f32x4_t dc[NG];
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const f32x4_t g = inseq(s0 + i) ? unpack(gg[m][i]) : zero4;
                if constexpr (SILU) {
                    // conv at s0+i from u at s0+i-3 .. s0+i (v index i .. i+3)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float conv = wt[0][r] * (al[i + 3] * vv[i + 3][r]) + wt[1][r] * (al[i + 2] * vv[i + 2][r]) +
                                           wt[2][r] * (al[i + 1] * vv[i + 1][r]) + wt[3][r] * (al[i] * vv[i][r]);
                        const float sg = sigmoid_b(conv);
                        dc[i][r] = g[r] * (sg + conv * sg * (1.f - sg));
                    }
                } else {
                    dc[i] = g;
                }
            }
#pragma unroll
            for (int k = 0; k < P; ++k) {
                const int t = s0 + k;
                if (t >= t1) break;
                // taps: u_{t-j} is v index k+3-j
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dw[j][r] += (al[k + 3 - j] * vv[k + 3 - j][r]) * dc[k][r];
                const f32x4_t g = SILU ? (inseq(t) ? unpack(gg[m][k]) : zero4) : zero4;
                float part = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float du = SILU ? g[r] : 0.f;
                    du += wt[0][r] * dc[k][r] + wt[1][r] * dc[k + 1][r] + wt[2][r] * dc[k + 2][r] +
                          wt[3][r] * dc[k + 3][r];
                    part += vv[k + 3][r] * du;
                    dv[k][r] += al[k + 3] * du;
                }
                part = wave_sum(part);
                if ((tid & 63) == 0) red[m][t - t0][tid >> 6] = part;
            }
        }
        if (live) {
#pragma unroll
            for (int k = 0; k < P; ++k)
                if (s0 + k < t1) store_bf16x4(a.dkv, (row0 + s0 + k) * a.dkv_ld + (int64_t)a.n_branches * d + c0, dv[k]);
        }
    }
    __syncthreads();
    // this stripe's dalpha of every position and branch, waves added in order
    for (int x = tid; x < BR * kConvPos; x += 256) {
        const int m = x / kConvPos, tt = x - m * kConvPos;
        if (t0 + tt >= t1) continue;
        const float s = (red[m][tt][0] + red[m][tt][1]) + (red[m][tt][2] + red[m][tt][3]);
        a.dalpha_part[((int64_t)m * a.n_stripes + blockIdx.z) * a.n_tok + row0 + t0 + tt] = s;
    }
    if (live) {
        float *dst = a.dconv_part + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * (int64_t)d * kc;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            for (int j = 0; j < kc; ++j) dst[(int64_t)(c0 + r) * kc + (kc - 1 - j)] = dw[j][r];
    }
}

// ---------------------------------------------------------------- gate and RMSNorms
// Workgroup (token chunk, branch, stripe); each thread four channels of
// kGateTok tokens.  With a = gh*h/rh, b = gk*k/rk, s = <a, b>/sqrt(d):
//   ds = dalpha alpha (1 - alpha), da = ds b/sqrt(d), db = ds a/sqrt(d)
//   dh = [dout] + (gh da - (h/rh) S/d)/rh,  dk = (gk db - (k/rk) S/d)/rk
// where S = <gh da, h/rh> = <gk db, k/rk> = ds s (both equal ds <a, b>/sqrt(d)).
__global__ __launch_bounds__(256) void bwd_gate_kernel(BwdArgs a) {
    __shared__ float sc[5][kGateTok];  // rh, rk, s, alpha, dalpha of the chunk's tokens
    const int m = blockIdx.y;
    const int64_t tb = (int64_t)blockIdx.x * kGateTok;
    const int d = a.d;
    const int tid = threadIdx.x;
    const int64_t plane = (int64_t)a.n_branches * a.n_tok;
    for (int x = tid; x < kGateTok; x += 256) {
        const int64_t t = tb + x;
        if (t >= a.n_tok) continue;
        const int64_t i = (int64_t)m * a.n_tok + t;
        sc[0][x] = a.stats[i];
        sc[1][x] = a.stats[plane + i];
        sc[2][x] = a.stats[2 * plane + i];
        sc[3][x] = a.stats[3 * plane + i];
        float dal = 0.f;
        for (int z = 0; z < a.n_stripes; ++z) dal += a.dalpha_part[((int64_t)m * a.n_stripes + z) * a.n_tok + t];
        sc[4][x] = dal;
    }
    __syncthreads();
    const int c0 = (blockIdx.z * 256 + tid) * 4;
    if (c0 >= d) return;
    const bool delta = (a.flags & ENGRAM_OUT_DELTA) != 0;
    const f32x4_t gh = *reinterpret_cast<const f32x4_t *>(pick_arg(a.gamma_h, m) + c0);
    const f32x4_t gk = *reinterpret_cast<const f32x4_t *>(pick_arg(a.gamma_k, m) + c0);
    const float inv_sqd = rsqrtf((float)d);
    f32x4_t dgh = {0.f, 0.f, 0.f, 0.f}, dgk = {0.f, 0.f, 0.f, 0.f};
    // tokens in groups of kGateGroup: the group's h, k and dout are all
    // requested (rows clamped into the tokens, raw bf16 widened at use)
    // before any arithmetic, then the tokens are taken in order, so the
    // gamma sums add them as a plain walk would
    const u32x2_t zero2 = {0u, 0u};
    for (int x0 = 0; x0 < kGateTok; x0 += kGateGroup) {
        u32x2_t hraw[kGateGroup], graw[kGateGroup];
        f32x4_t kvs[kGateGroup];
#pragma unroll
        for (int u = 0; u < kGateGroup; ++u) {
            const int64_t t = min(tb + x0 + u, a.n_tok - 1);
            const int64_t hi = ((int64_t)m * a.n_tok + t) * d + c0;
            hraw[u] = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(a.h) + hi);
            kvs[u] = *reinterpret_cast<const f32x4_t *>(a.kv + t * a.kv_ld + (int64_t)m * d + c0);
            graw[u] = delta ? zero2 : *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(a.dout) + hi);
        }
#pragma unroll
        for (int u = 0; u < kGateGroup; ++u) {
            const int x = x0 + u;
            const int64_t t = tb + x;
            if (t >= a.n_tok) break;
            const float rh = sc[0][x], rk = sc[1][x], s = sc[2][x], al = sc[3][x];
            const float ds = sc[4][x] * al * (1.f - al);
            const float corr = ds * s / (float)d;
            const int64_t hi = ((int64_t)m * a.n_tok + t) * d + c0;
            const f32x4_t hv = {bf16_to_f32(hraw[u][0] & 0xFFFFu), bf16_to_f32(hraw[u][0] >> 16),
                                bf16_to_f32(hraw[u][1] & 0xFFFFu), bf16_to_f32(hraw[u][1] >> 16)};
            const f32x4_t g = {bf16_to_f32(graw[u][0] & 0xFFFFu), bf16_to_f32(graw[u][0] >> 16),
                               bf16_to_f32(graw[u][1] & 0xFFFFu), bf16_to_f32(graw[u][1] >> 16)};
            const f32x4_t kv = kvs[u];
            f32x4_t dh, dk;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float hn = hv[r] / rh, kn = kv[r] / rk;
                const float da = ds * (gk[r] * kn) * inv_sqd;
                const float db = ds * (gh[r] * hn) * inv_sqd;
                dgh[r] += da * hn;
                dgk[r] += db * kn;
                dh[r] = g[r] + (gh[r] * da - hn * corr) / rh;
                dk[r] = (gk[r] * db - kn * corr) / rk;
            }
            store_bf16x4(a.dh, hi, dh);
            store_bf16x4(a.dkv, t * a.dkv_ld + (int64_t)m * d + c0, dk);
        }
    }
    const int64_t pr = ((int64_t)m * gridDim.x + blockIdx.x) * d + c0;
    *reinterpret_cast<f32x4_t *>(a.dg_part + pr) = dgh;
    *reinterpret_cast<f32x4_t *>(a.dg_part + (int64_t)a.n_branches * gridDim.x * d + pr) = dgk;
}

// Sums over the rows of in[g][rows][width], in a fixed order, in two
// stages.  Stage 1: slab s of S holds rows [s*rows/S, (s+1)*rows/S); four
// threads per column each add every fourth row of the slab, ascending, and
// the four sums are added in thread order into part[g][s][i].
__global__ __launch_bounds__(256) void bwd_sum_slabs_kernel(const float *in, int64_t rows, int64_t width, int32_t S,
                                                            float *part) {
    __shared__ float red[4][64];
    const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * 64 + c;
    const int64_t g = blockIdx.y, s = blockIdx.z;
    const int64_t r0 = s * rows / S, r1 = (s + 1) * rows / S;
    float acc = 0.f;
    if (i < width) {
        const float *p = in + g * rows * width + i;
#pragma unroll 4
        for (int64_t r = r0 + q; r < r1; r += 4) acc += p[r * width];
    }
    red[q][c] = acc;
    __syncthreads();
    if (q == 0 && i < width) part[(g * S + s) * width + i] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// Stage 2 (and the split-K sum of a contraction): out[g][i] = sum over
// s = 0..S-1, ascending, of part[g][s][i].
__global__ __launch_bounds__(256) void bwd_sum_parts_kernel(const float *part, int64_t groups, int64_t width,
                                                            int32_t S, float *out) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= groups * width) return;
    const int64_t gi = x / width, i = x - gi * width;
    const float *p = part + gi * S * width + i;
    float s = 0.f;
#pragma unroll 16
    for (int k = 0; k < S; ++k) s += p[k * width];
    out[x] = s;
}

// ---------------------------------------------------------------- table rows
// Item i = tau * n_tok + t: key tau << row_bits | idx[t][tau], value t.
template <typename KeyT>
__global__ __launch_bounds__(256) void bwd_keys_kernel(const uint32_t *idx, int64_t n_tok, int32_t n_tables,
                                                       int32_t row_bits, KeyT *keys, uint32_t *vals) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_tok * n_tables) return;
    const int64_t tau = i / n_tok, t = i - tau * n_tok;
    keys[i] = (KeyT)(((uint64_t)tau << row_bits) | idx[t * n_tables + tau]);
    vals[i] = (uint32_t)t;
}

// Stable LSD radix sort of the keys by their row bits, one table at a time.
// The keys arrive grouped by table (item tau * n_tok + t is token t's key in
// table tau, tokens ascending), so sorting each table's segment by row is
// sorting by (table, row), and stability keeps the tokens of one row in
// ascending order.  A pass takes `bits` digit bits from `shift` up:
//   sort_count_kernel    digit counts of every block of kSortItems items
//   sort_scan_kernel     per table, exclusive offsets in (digit, block) order
//   sort_scatter_kernel  each wave walks its quarter of the block in order,
//                        64 items at a time; a lane's rank among the lanes
//                        holding its digit comes from `bits` ballots, so the
//                        order of the items is kept without atomics
constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = 2048;  // per block: 512 per wave
constexpr int kSortMaxBits = 11;

// lanes of the wave (among those with `valid`) whose digit equals this lane's
__device__ __forceinline__ uint64_t digit_peers(uint32_t digit, int bits, bool valid) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
        const bool set = (digit >> b) & 1u;
        const uint64_t m = __ballot(set);
        peers &= set ? m : ~m;
    }
    return peers;
}

// Each wave owns a contiguous quarter of its block's items, kSortGroups
// groups of 64, and loads all of them before it ranks any (one memory round
// trip per kernel instead of one per group).
constexpr int kSortGroups = kSortItems / kSortWaves / 64;

template <typename KeyT>
__device__ __forceinline__ void sort_load(const KeyT *k, int wlo, int whi, int lane, KeyT (&key)[kSortGroups]) {
#pragma unroll
    for (int g = 0; g < kSortGroups; ++g) {
        const int i = wlo + 64 * g + lane;
        key[g] = i < whi ? k[i] : (KeyT)0;
    }
}

template <typename KeyT>
__global__ __launch_bounds__(kSortThreads) void sort_count_kernel(const KeyT *keys, int64_t seg, int32_t nbpt,
                                                                  int32_t shift, int32_t bits, uint32_t *hist) {
    __shared__ uint32_t cnt[1 << kSortMaxBits];
    const int nd = 1 << bits;
    const int tau = blockIdx.y, blk = blockIdx.x;
    const int64_t lo = (int64_t)blk * kSortItems;
    const int n = (int)min<int64_t>(kSortItems, seg - lo);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wlo = w * (kSortItems / kSortWaves), whi = min(wlo + kSortItems / kSortWaves, n);
    KeyT key[kSortGroups];
    sort_load(keys + (int64_t)tau * seg + lo, wlo, whi, lane, key);
    for (int i = threadIdx.x; i < nd; i += kSortThreads) cnt[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kSortGroups; ++g) {
        const bool valid = wlo + 64 * g + lane < whi;
        const uint32_t digit = (uint32_t)(key[g] >> shift) & (uint32_t)(nd - 1);
        const uint64_t peers = digit_peers(digit, bits, valid);
        // the lowest lane of each digit adds the lanes that share it
        if (valid && (peers & ((1ull << lane) - 1ull)) == 0ull) atomicAdd(&cnt[digit], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    uint32_t *h = hist + (int64_t)tau * nd * nbpt;
    for (int dg = threadIdx.x; dg < nd; dg += kSortThreads) h[(int64_t)dg * nbpt + blk] = cnt[dg];
}

// One workgroup of 16 waves per table: hist[tau][0..per_table) becomes its
// exclusive prefix sum, in chunks of 16 x kScanRows x 64 counts.  Wave w
// takes a contiguous kScanRows x 64 of the chunk and loads it row by row
// (lane l of row j holds count 64 j + l: every access is coalesced); each row
// is scanned across the lanes and carried to the next, the waves' totals are
// scanned in LDS, and the prefixes go back the way they came.
constexpr int kScanRows = 16;

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

__global__ __launch_bounds__(1024) void sort_scan_kernel(uint32_t *hist, int64_t per_table) {
    __shared__ uint32_t wtot[16];
    uint32_t *h = hist + (int64_t)blockIdx.x * per_table;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t carry = 0u;  // total of the earlier chunks
    for (int64_t c0 = 0; c0 < per_table; c0 += 16 * kScanRows * 64) {
        const int64_t base = c0 + (int64_t)w * kScanRows * 64 + lane;
        uint32_t x[kScanRows];
#pragma unroll
        for (int j = 0; j < kScanRows; ++j) x[j] = base + 64 * j < per_table ? h[base + 64 * j] : 0u;
        uint32_t run = 0u;  // this wave's total so far
#pragma unroll
        for (int j = 0; j < kScanRows; ++j) {
            const uint32_t incl = wave_incl_scan(x[j], lane);
            const uint32_t tot = __shfl(incl, 63);
            x[j] = run + incl - x[j];
            run += tot;
        }
        if (lane == 0) wtot[w] = run;
        __syncthreads();
        uint32_t woff = carry, all = 0u;
        for (int ww = 0; ww < 16; ++ww) {
            const uint32_t t = wtot[ww];
            woff += ww < w ? t : 0u;
            all += t;
        }
#pragma unroll
        for (int j = 0; j < kScanRows; ++j)
            if (base + 64 * j < per_table) h[base + 64 * j] = woff + x[j];
        carry += all;
        __syncthreads();  // wtot is rewritten by the next chunk
    }
}

template <typename KeyT>
__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(const KeyT *kin, const uint32_t *vin, KeyT *kout,
                                                                    uint32_t *vout, int64_t seg, int32_t nbpt,
                                                                    int32_t shift, int32_t bits,
                                                                    const uint32_t *hist) {
    __shared__ uint32_t wbase[kSortWaves][1 << kSortMaxBits];
    const int nd = 1 << bits;
    const int tau = blockIdx.y, blk = blockIdx.x;
    const int64_t lo = (int64_t)blk * kSortItems;
    const int n = (int)min<int64_t>(kSortItems, seg - lo);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t below = (1ull << lane) - 1ull;
    const int wlo = w * (kSortItems / kSortWaves), whi = min(wlo + kSortItems / kSortWaves, n);
    KeyT key[kSortGroups];
    uint32_t val[kSortGroups];
    sort_load(kin + (int64_t)tau * seg + lo, wlo, whi, lane, key);
    sort_load(vin + (int64_t)tau * seg + lo, wlo, whi, lane, val);
    for (int i = threadIdx.x; i < kSortWaves * nd; i += kSortThreads) wbase[i / nd][i % nd] = 0u;
    __syncthreads();
    // digit counts of each wave's quarter
    uint64_t peers[kSortGroups];
#pragma unroll
    for (int g = 0; g < kSortGroups; ++g) {
        const bool valid = wlo + 64 * g + lane < whi;
        const uint32_t digit = (uint32_t)(key[g] >> shift) & (uint32_t)(nd - 1);
        peers[g] = digit_peers(digit, bits, valid);
        if (valid && (peers[g] & below) == 0ull) wbase[w][digit] += (uint32_t)__popcll(peers[g]);
    }
    __syncthreads();
    // first output slot of each (wave, digit): the block's offset plus the
    // counts of the earlier waves
    const uint32_t *h = hist + (int64_t)tau * nd * nbpt;
    for (int dg = threadIdx.x; dg < nd; dg += kSortThreads) {
        uint32_t run = h[(int64_t)dg * nbpt + blk];
#pragma unroll
        for (int ww = 0; ww < kSortWaves; ++ww) {
            const uint32_t c = wbase[ww][dg];
            wbase[ww][dg] = run;
            run += c;
        }
    }
    __syncthreads();
    KeyT *ko = kout + (int64_t)tau * seg;
    uint32_t *vo = vout + (int64_t)tau * seg;
#pragma unroll
    for (int g = 0; g < kSortGroups; ++g) {
        const bool valid = wlo + 64 * g + lane < whi;
        const uint32_t digit = (uint32_t)(key[g] >> shift) & (uint32_t)(nd - 1);
        const uint32_t pos = wbase[w][digit] + (uint32_t)__popcll(peers[g] & below);
        if (valid) {
            ko[pos] = key[g];
            vo[pos] = val[g];
        }
        // every peer has read the base (the wave's LDS accesses complete in
        // order); the highest peer moves it past the group
        if (valid && (peers[g] >> lane) == 1ull) wbase[w][digit] = pos + 1u;
    }
}

// Run heads of the sorted keys (head[i] = 1 where a new key starts) and
// their inclusive prefix count incl[i], the number of heads in [0, i]:
//   bwd_heads_count_kernel  head flags; heads per block of kHeadItems items
//   sort_scan_kernel        (one workgroup) exclusive offsets of the blocks
//   bwd_heads_incl_kernel   each wave ranks 64 items at a time by ballot and
//                           popcount, offset by its block's and waves' counts
// Wave w of a block owns items [w * kHeadItems / 4, (w + 1) * kHeadItems / 4).
constexpr int kHeadItems = 2048;
constexpr int kHeadRows = kHeadItems / 4 / 64;  // rows of 64 per wave

template <typename KeyT>
__global__ __launch_bounds__(256) void bwd_heads_count_kernel(const KeyT *keys, int64_t n, uint32_t *head,
                                                              uint32_t *bcount) {
    __shared__ uint32_t wtot[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t base = (int64_t)blockIdx.x * kHeadItems + (int64_t)w * (kHeadItems / 4) + lane;
    uint32_t cnt = 0u;
#pragma unroll
    for (int r = 0; r < kHeadRows; ++r) {
        const int64_t i = base + 64 * r;
        if (i < n) {
            const uint32_t hd = (i == 0 || keys[i] != keys[i - 1]) ? 1u : 0u;
            head[i] = hd;
            cnt += hd;
        }
    }
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) wtot[w] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) bcount[blockIdx.x] = wtot[0] + wtot[1] + wtot[2] + wtot[3];
}

__global__ __launch_bounds__(256) void bwd_heads_incl_kernel(const uint32_t *head, int64_t n,
                                                             const uint32_t *boff, uint32_t *incl) {
    __shared__ uint32_t wtot[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t base = (int64_t)blockIdx.x * kHeadItems + (int64_t)w * (kHeadItems / 4);
    const uint64_t le = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);  // lanes 0..lane
    uint32_t hd[kHeadRows];
    uint32_t tot = 0u;
#pragma unroll
    for (int r = 0; r < kHeadRows; ++r) {
        const int64_t i = base + 64 * r + lane;
        hd[r] = i < n ? head[i] : 0u;
        tot += (uint32_t)__popcll(__ballot(hd[r] != 0u));
    }
    if (lane == 0) wtot[w] = tot;
    __syncthreads();
    uint32_t run = boff[blockIdx.x];
    for (int ww = 0; ww < w; ++ww) run += wtot[ww];
#pragma unroll
    for (int r = 0; r < kHeadRows; ++r) {
        const uint64_t m = __ballot(hd[r] != 0u);
        const int64_t i = base + 64 * r + lane;
        if (i < n) incl[i] = run + (uint32_t)__popcll(m & le);
        run += (uint32_t)__popcll(m);
    }
}

// Per-table row gradients as a segmented sum over the sorted items, in two
// passes over fixed 64-item chunks, one wave per chunk.  Pass 1 adds the
// chunk's dE slices in item order (tokens ascending within each run: the sort
// is stable).  A run that starts and ends inside the chunk is written to its
// row slot directly; the part of a run that began in an earlier chunk goes
// to lead[chunk], the part of the chunk's last run that continues past the
// chunk goes to tail[chunk] (with its slot and row).  Pass 2 adds, for every
// chunk with a tail, the lead parts of the following chunks in chunk order.
// The order of every sum depends only on the sorted items, so the result is
// the same on every run.
constexpr int kRowChunk = 64;
constexpr uint32_t kChunkHasHead = 1u, kChunkLead = 2u, kChunkTail = 4u;

template <int NQ, typename KeyT>  // head_dim <= 64 * NQ
__global__ __launch_bounds__(256) void bwd_row_chunks_kernel(const KeyT *keys, uint64_t row_mask, const uint32_t *vals,
                                                             const uint32_t *head, const uint32_t *incl,
                                                             const float *demb, int64_t n_tok, int32_t n_tables,
                                                             int32_t head_dim, uint32_t *row_ids, float *row_grads,
                                                             int32_t *row_counts, float *lead, float *tail,
                                                             uint32_t *cflags, uint32_t *tinfo) {
    const int64_t n = n_tok * n_tables;
    const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t base = c * kRowChunk;
    if (base >= n) return;
    const int cnt = (int)min((int64_t)kRowChunk, n - base);
    const int64_t j = base + lane;
    const bool in = lane < cnt;
    uint32_t my_off = 0, my_slot = 0, my_row = 0;
    bool my_head = false;
    if (in) {
        const int64_t tau = j / n_tok, first = tau * n_tok;
        const uint32_t inc = incl[j];
        my_head = head[j] != 0;
        my_row = (uint32_t)(keys[j] & (KeyT)row_mask);
        my_slot = (uint32_t)(first + inc - incl[first]);
        my_off = vals[j] * (uint32_t)(n_tables * head_dim) + (uint32_t)(tau * head_dim);
        if (j == first) row_counts[tau] = (int32_t)(incl[first + n_tok - 1] - inc + 1);
    }
    const uint64_t hmask = __ballot(my_head);
    const bool next_head = (base + cnt >= n) || head[base + cnt] != 0;
    bool has_tail = false;
    float acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
    for (int k0 = 0; k0 < cnt; k0 += 8) {
        float v[8][NQ];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = min(k0 + u, cnt - 1);
            const float *src = demb + (uint32_t)__builtin_amdgcn_readlane((int)my_off, k);
#pragma unroll
            for (int q = 0; q < NQ; ++q) v[u][q] = (lane + 64 * q < head_dim) ? src[lane + 64 * q] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = k0 + u;
            if (k >= cnt) break;
#pragma unroll
            for (int q = 0; q < NQ; ++q) acc[q] += v[u][q];
            const bool last = k == cnt - 1;
            const bool ends = last ? next_head : ((hmask >> (k + 1)) & 1ull) != 0;
            if (!(ends || last)) continue;
            const bool started_here = (hmask & ((2ull << k) - 1ull)) != 0;
            float *dst;
            if (!started_here) {
                dst = lead + c * head_dim;
            } else {
                const uint32_t slot = (uint32_t)__builtin_amdgcn_readlane((int)my_slot, k);
                const uint32_t row = (uint32_t)__builtin_amdgcn_readlane((int)my_row, k);
                if (ends) {
                    dst = row_grads + (int64_t)slot * head_dim;
                    if (lane == 0) row_ids[slot] = row;
                } else {
                    dst = tail + c * head_dim;
                    has_tail = true;
                    if (lane == 0) {
                        tinfo[2 * c] = slot;
                        tinfo[2 * c + 1] = row;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (lane + 64 * q < head_dim) dst[lane + 64 * q] = acc[q];
                acc[q] = 0.f;
            }
        }
    }
    if (lane == 0)
        cflags[c] = (hmask ? kChunkHasHead : 0u) | ((hmask & 1ull) ? 0u : kChunkLead) | (has_tail ? kChunkTail : 0u);
}

__global__ __launch_bounds__(256) void bwd_row_chain_kernel(const float *lead, const float *tail,
                                                            const uint32_t *cflags, const uint32_t *tinfo,
                                                            int64_t n_chunks, int32_t head_dim, uint32_t *row_ids,
                                                            float *row_grads) {
    const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (c >= n_chunks || !(cflags[c] & kChunkTail)) return;
    float acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = (lane + 64 * q < head_dim) ? tail[c * head_dim + lane + 64 * q] : 0.f;
    for (int64_t k = c + 1; k < n_chunks; ++k) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + 64 * q < head_dim) acc[q] += lead[k * head_dim + lane + 64 * q];
        if ((cflags[k] & kChunkHasHead) || k + 1 == n_chunks || !(cflags[k + 1] & kChunkLead)) break;
    }
    const uint32_t slot = tinfo[2 * c];
    if (lane == 0) row_ids[slot] = tinfo[2 * c + 1];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < head_dim) row_grads[(int64_t)slot * head_dim + lane + 64 * q] = acc[q];
}

}  // namespace

void launch_bwd_gate_stats(const BwdArgs &a, hipStream_t s) {
    launch_kernel(bwd_gate_stats_kernel, dim3((unsigned)((a.n_tok + 255) / 256), a.n_branches), dim3(256), s, a);
}

void launch_bwd_conv(const BwdArgs &a, hipStream_t s) {
    const dim3 grid((a.seqlen + kConvPos - 1) / kConvPos, a.batch, a.n_stripes);
    const bool silu = a.conv_mode == ENGRAM_CONV_SILU_SKIP;
#define ENGRAM_BWD_CONV(BR)                                                                     \
    do {                                                                                        \
        if (silu)                                                                               \
            launch_kernel((bwd_conv_kernel<BR, true>), grid, dim3(256), s, a);                  \
        else                                                                                    \
            launch_kernel((bwd_conv_kernel<BR, false>), grid, dim3(256), s, a);                 \
    } while (0)
    switch (a.n_branches) {
        case 1: ENGRAM_BWD_CONV(1); break;
        case 2: ENGRAM_BWD_CONV(2); break;
        case 3: ENGRAM_BWD_CONV(3); break;
        default: ENGRAM_BWD_CONV(4); break;
    }
#undef ENGRAM_BWD_CONV
}

int32_t bwd_conv_blocks(int32_t batch, int32_t seqlen) { return batch * ((seqlen + kConvPos - 1) / kConvPos); }
int32_t bwd_gate_chunks(int64_t n_tok) { return (int32_t)((n_tok + kGateTok - 1) / kGateTok); }

void launch_bwd_gate(const BwdArgs &a, hipStream_t s) {
    launch_kernel(bwd_gate_kernel, dim3((unsigned)bwd_gate_chunks(a.n_tok), a.n_branches, a.n_stripes), dim3(256),
                  s, a);
}

int32_t bwd_sum_slabs(int64_t rows) { return (int32_t)std::min<int64_t>(64, rows); }

void launch_bwd_sum_rows(const float *in, int64_t groups, int64_t rows, int64_t width, float *part, float *out,
                         hipStream_t s) {
    const int32_t S = bwd_sum_slabs(rows);
    launch_kernel(bwd_sum_slabs_kernel, dim3((unsigned)((width + 63) / 64), (unsigned)groups, (unsigned)S),
                  dim3(256), s, in, rows, width, S, part);
    launch_bwd_sum_parts(part, groups, width, S, out, s);
}

void launch_bwd_sum_parts(const float *part, int64_t groups, int64_t width, int32_t S, float *out, hipStream_t s) {
    const int64_t n = groups * width;
    launch_kernel(bwd_sum_parts_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, part, groups, width, S, out);
}

int64_t bwd_row_chunks(int64_t n_items) { return (n_items + kRowChunk - 1) / kRowChunk; }

namespace {
size_t sort_hist_bytes(int64_t n_items) {
    // (digits x blocks) counts per table: at most 2^kSortMaxBits per block
    // of kSortItems items, plus one partial block per table (<= 32 tables)
    return (size_t)(n_items + (int64_t)32 * kSortItems) * 4u;
}

size_t table_temp_bytes(int64_t n_items) {
    // the sort's histograms, then the run heads' per-block counts
    const size_t head_blocks = (size_t)((n_items + kHeadItems - 1) / kHeadItems) * 4u;
    return std::max(head_blocks, sort_hist_bytes(n_items));
}

template <typename KeyT>
hipError_t table_grad(const BwdTableArgs &t, int32_t row_bits, hipStream_t s) {
    const int64_t n = t.n_tok * t.n_tables;
    // passes of at most kSortMaxBits digit bits over the row bits; the keys
    // start in the buffer that makes the last pass end in keys_out
    const int passes = (row_bits + kSortMaxBits - 1) / kSortMaxBits;
    const int bits = (row_bits + passes - 1) / passes;
    KeyT *kb[2] = {static_cast<KeyT *>(t.keys_in), static_cast<KeyT *>(t.keys_out)};
    uint32_t *vb[2] = {t.vals_in, t.vals_out};
    int cur = passes % 2 == 0 ? 1 : 0;
    launch_kernel(bwd_keys_kernel<KeyT>, dim3((unsigned)((n + 255) / 256)), dim3(256), s, t.idx, t.n_tok,
                  t.n_tables, row_bits, kb[cur], vb[cur]);
    const int32_t nbpt = (int32_t)((t.n_tok + kSortItems - 1) / kSortItems);
    uint32_t *hist = static_cast<uint32_t *>(t.temp);
    const dim3 sgrid((unsigned)nbpt, (unsigned)t.n_tables);
    for (int p = 0, shift = 0; p < passes; ++p, shift += bits) {
        const int pb = std::min(bits, row_bits - shift);
        launch_kernel(sort_count_kernel<KeyT>, sgrid, dim3(kSortThreads), s, kb[cur], t.n_tok, nbpt, shift, pb, hist);
        launch_kernel(sort_scan_kernel, dim3((unsigned)t.n_tables), dim3(1024), s, hist,
                      (int64_t)nbpt << pb);
        launch_kernel(sort_scatter_kernel<KeyT>, sgrid, dim3(kSortThreads), s, kb[cur], vb[cur], kb[cur ^ 1],
                      vb[cur ^ 1], t.n_tok, nbpt, shift, pb, hist);
        cur ^= 1;
    }
    KeyT *keys_out = kb[1];
    const int64_t head_blocks = (n + kHeadItems - 1) / kHeadItems;
    uint32_t *bcount = static_cast<uint32_t *>(t.temp);  // the sort is done with hist
    launch_kernel(bwd_heads_count_kernel<KeyT>, dim3((unsigned)head_blocks), dim3(256), s, keys_out, n, t.head,
                  bcount);
    launch_kernel(sort_scan_kernel, dim3(1), dim3(1024), s, bcount, head_blocks);
    launch_kernel(bwd_heads_incl_kernel, dim3((unsigned)head_blocks), dim3(256), s, t.head, n, bcount, t.incl);
    const int64_t chunks = bwd_row_chunks(n);
    const dim3 grid((unsigned)((chunks + 3) / 4));
    const uint64_t row_mask = (row_bits >= 64) ? ~0ull : ((1ull << row_bits) - 1ull);
#define ENGRAM_ROW_CHUNKS(NQ)                                                                                   \
    launch_kernel((bwd_row_chunks_kernel<NQ, KeyT>), grid, dim3(256), s, keys_out, row_mask, t.vals_out, t.head, \
                  t.incl, t.demb, t.n_tok, t.n_tables, t.head_dim, t.row_ids, t.row_grads, t.row_counts, t.lead,  \
                  t.tail, t.cflags, t.tinfo)
    if (t.head_dim <= 64)
        ENGRAM_ROW_CHUNKS(1);
    else if (t.head_dim <= 128)
        ENGRAM_ROW_CHUNKS(2);
    else
        ENGRAM_ROW_CHUNKS(4);
#undef ENGRAM_ROW_CHUNKS
    launch_kernel(bwd_row_chain_kernel, grid, dim3(256), s, t.lead, t.tail, t.cflags, t.tinfo, chunks, t.head_dim,
                  t.row_ids, t.row_grads);
    return hipGetLastError();
}
}  // namespace

size_t bwd_table_temp_bytes(int64_t n_items) { return table_temp_bytes(n_items); }

hipError_t launch_bwd_table_grad(const BwdTableArgs &t, hipStream_t s) {
    // key = tau << row_bits | row, in 32 bits when the widest table and the
    // table count fit there
    uint32_t max_row = 0;
    for (int tau = 0; tau < t.n_tables; ++tau) max_row = std::max(max_row, t.table_rows[tau] - 1u);
    int32_t row_bits = 1, tau_bits = 0;
    while (row_bits < 32 && (max_row >> row_bits) != 0) ++row_bits;
    while ((1 << tau_bits) < t.n_tables) ++tau_bits;
    const int32_t key_bits = row_bits + tau_bits;
    if (key_bits <= 32) return table_grad<uint32_t>(t, row_bits, s);
    return table_grad<uint64_t>(t, row_bits, s);
}

}  // namespace engram
