// fuse.hip -- the gate, the seam rows of the fused value projection and, for
// short chunks and the fp32 path, the rest of Engram's fusion step on gfx950 ([club] 1.(2) 上下文感知的门控机制, last two
// bullets; [csdn] Engram 到底怎么工作的, third and fourth steps).
//
// gate_kernel: the scalar gate per token and branch from the partial sums the
// projection kernel left behind (one thread per token, the partial index
// summed in a fixed order, so every path gets the same bits).
//
// fuse_kernel: the gated value u = alpha * v, the short depthwise causal
// convolution and the residual into the hidden state.  HBM-bound: it reads v
// (fp32) once, h once per branch and writes out once per branch.  A block
// owns kPos consecutive positions of one sequence and a stripe of channels;
// each thread owns 4 channels (one 16-byte fp32 vector of v) and walks the
// positions in order, keeping the last three gated values of every branch in
// registers, so no gated value is ever written to memory.  Loads for a group
// of positions are issued before any of their arithmetic.  The three values
// before the block's first position are recomputed from v (or taken from the
// carried conv state at the sequence start).  Those values, the first
// group's v and h and the gate partials (staged in LDS by the whole block)
// and the conv taps are all requested before any of them is used: at decode
// the kernel makes one round trip to memory before it stores.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kPos = kFusePositions;
constexpr int kVec = 4;

// Four values in their stored form: 8 bytes for bf16, 16 for fp32.
template <bool BF16>
struct Raw4 {
    u32x4_t w;
    __device__ __forceinline__ void load(const void *base, int64_t off) {
        if constexpr (BF16) {
            const u32x2_t x = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(base) + off);
            w[0] = x[0];
            w[1] = x[1];
        } else {
            w = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const float *>(base) + off);
        }
    }
    __device__ __forceinline__ float get(int c) const {
        if constexpr (BF16) {
            const uint32_t x = w[c >> 1];
            return bf16_to_f32((c & 1) ? (x >> 16) : (x & 0xFFFFu));
        } else {
            return __uint_as_float(w[c]);
        }
    }
    static __device__ __forceinline__ void store(void *base, int64_t off, const float (&x)[kVec]) {
        if constexpr (BF16) {
            *reinterpret_cast<u32x2_t *>(reinterpret_cast<uint16_t *>(base) + off) =
                u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        } else {
            *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(base) + off) = f32x4_t{x[0], x[1], x[2], x[3]};
        }
    }
};

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

// Four consecutive values of a carried conv-state row (element offset off):
// fp32, or bf16 widened exactly.
__device__ __forceinline__ f32x4_t load_state4(const void *state, bool bf16, int64_t off) {
    if (bf16) {
        const u32x2_t x = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(state) + off);
        return f32x4_t{bf16_to_f32(x[0] & 0xFFFFu), bf16_to_f32(x[0] >> 16), bf16_to_f32(x[1] & 0xFFFFu),
                       bf16_to_f32(x[1] >> 16)};
    }
    return *reinterpret_cast<const f32x4_t *>(reinterpret_cast<const float *>(state) + off);
}

// The gate from the three sums over d of h*gamma_h*gamma_k*k, k^2 and h^2.
__device__ __forceinline__ float gate_finish(float s_hk, float s_kk, float s_hh, int d, float eps) {
    const float inv_d = 1.f / (float)d;
    const float rh = sqrtf(s_hh * inv_d + eps);
    const float rk = sqrtf(s_kk * inv_d + eps);
    return sigmoidf_(s_hk / (rh * rk) * rsqrtf((float)d));
}

// The gate of token t, branch m, from the n_parts partial sums, added in
// part order.  Every path adds the parts in this order and finishes with
// gate_finish, so every path gets the same bits.
__device__ __forceinline__ float gate_value(const float *partials, int m, int n_parts, int64_t n_tok, int64_t t,
                                            int d, float eps) {
    const float *pp = partials + (int64_t)m * n_parts * 3 * n_tok + t;
    float s_hk = 0.f, s_kk = 0.f, s_hh = 0.f;
#pragma unroll 8
    for (int q = 0; q < n_parts; ++q) {
        s_hk += pp[(3 * q + 0) * n_tok];
        s_kk += pp[(3 * q + 1) * n_tok];
        s_hh += pp[(3 * q + 2) * n_tok];
    }
    return gate_finish(s_hk, s_kk, s_hh, d, eps);
}

__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int m = blockIdx.y;
    if (a.ctx.prev_ctx && m == 0 && t < a.batch) ctx_update_one(a.ctx, (int32_t)t, a.seqlen);
    if (t >= a.n_tok) return;
    a.alpha[m * a.n_tok + t] = gate_value(a.partials, m, a.n_parts, a.n_tok, t, a.d, a.eps);
}

// Conv taps of 4 channels, wt[j][c] multiplying u_{t-j} of channel c0 + c
// (the weight stored at index K_c-1-j; zero for j >= K_c is chosen at use).
// TAP4: K_c = 4 and the taps 16-byte aligned, so a channel's four taps are
// one load (else one load per tap; either way the lanes are 16 K_c bytes
// apart).
template <bool TAP4>
__device__ __forceinline__ void load_taps(const float *conv_w, int kc, int c0, float (&wt)[4][kVec]) {
    if constexpr (TAP4) {
#pragma unroll
        for (int c = 0; c < kVec; ++c) {
            const f32x4_t w4 = *reinterpret_cast<const f32x4_t *>(conv_w + (int64_t)(c0 + c) * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) wt[j][c] = w4[3 - j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < kVec; ++c) wt[j][c] = conv_w[(int64_t)(c0 + c) * kc + max(kc - 1 - j, 0)];
    }
}

constexpr int kPartCap = 4096;  // gate partials staged in LDS per round
// Threads per workgroup at most: the channel quads of a token are split into
// the fewest workgroups of at most five waves (d = 2560: two of 320 threads,
// where 256-thread workgroups leave a third one half empty).
constexpr int kFuseMaxThreads = 320;

// SBF16: the carried conv state is bf16 (else fp32).  A compile-time choice:
// with a runtime one the compiler widens each bf16 row inside its branch and
// waits for that load alone, one memory round trip per state row.
// TAP4: K_c = 4 with 16-byte aligned taps (one load per channel).  ONE: one
// position per sequence (a decode step): no earlier rows of v to read and one
// position per group, so no load is made twice.
template <bool BF16, int BR, bool SBF16, bool TAP4, bool ONE>
__global__ __launch_bounds__(kFuseMaxThreads) void fuse_kernel(FuseArgs a) {
    __shared__ float alpha_s[BR][kPos + 3];
    __shared__ float sums_s[3][BR * (kPos + 3)];
    __shared__ float part_s[kPartCap];
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kPos;
    const int t1 = min(t0 + kPos, a.seqlen);
    const int64_t n_tok = (int64_t)a.batch * a.seqlen;
    const int64_t row0 = (int64_t)b * a.seqlen;
    const int d = a.d;
    const int tid = threadIdx.x;
    const int c0 = (blockIdx.z * blockDim.x + tid) * kVec;
    const bool live = c0 < d;
    const int kc = a.conv_k;

    if (a.ctx.prev_ctx && blockIdx.x == 0 && blockIdx.z == 0 && tid == 0) ctx_update_one(a.ctx, b, a.seqlen);

    // Gates of positions pa .. t1-1 (the block's and up to three before it).
    // The whole block stages the partial sums in LDS, as many parts per
    // round as fit (all of them at decode sizes); one thread per (branch,
    // position) then adds them in part order, as gate_value does.  Staged
    // layout: x = ((qq * BR + m) * 3 + k) * npos + pi.
    const int pa = max(t0 - 3, 0);
    const int npos = t1 - pa;
    const int n_sum = BR * npos;
    const int per_part = 3 * n_sum;
    const int q_round = max(1, kPartCap / per_part);
    auto part_at = [&](int x, int q0) -> int64_t {
        const int pi = x % npos;
        const int r = x / npos;
        const int k = r % 3;
        const int mq = r / 3;
        const int m = mq % BR, qq = mq / BR;
        return (((int64_t)m * a.n_parts + q0 + qq) * 3 + k) * n_tok + row0 + pa + pi;
    };
    // The first round's partial sums, up to kPre per thread, are requested
    // before anything else: waiting for them then waits for no other load,
    // and the gate is taken while the rest is still in flight.
    constexpr int kPre = 2;
    const int n_first = min(q_round, a.n_parts) * per_part;
    float pre[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) pre[i] = a.partials[part_at(min(tid + i * (int)blockDim.x, n_first - 1), 0)];

    // Everything this thread reads that does not depend on the gate is
    // requested next: the three values before t0 (v of earlier positions,
    // or the carried state at the sequence start) and the first group's v
    // and h.
    // Every one of these loads is issued unconditionally: lanes that need no
    // value read a valid element, and the choice between it and zero is made
    // where the value is used, past the barriers below, so the compiler can
    // neither sink a load into a branch nor wait for it early, and the
    // partial sums above wait for none of them.  State rows stay in their
    // stored form until first use.
    const int cc0 = live ? c0 : 0;
    const void *sbase = a.conv_state ? a.conv_state : static_cast<const void *>(a.v);
    f32x4_t vprev[3];
    Raw4<SBF16> sprev[BR][3];
    bool vprev_ok[3], sprev_ok[3];
#pragma unroll
    for (int s = 1; s <= 3; ++s) {
        const int p = t0 - s;
        if constexpr (ONE) {
            vprev[s - 1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            vprev_ok[s - 1] = false;
        } else {
            vprev[s - 1] = *reinterpret_cast<const f32x4_t *>(a.v + (row0 + max(p, 0)) * d + cc0);
            vprev_ok[s - 1] = live && p >= 0;
        }
        const bool need = live && p < 0 && a.conv_state && s <= kc - 1;
        sprev_ok[s - 1] = need;
#pragma unroll
        for (int m = 0; m < BR; ++m)
            sprev[m][s - 1].load(sbase, need ? (((int64_t)m * a.batch + b) * (kc - 1) + (kc - 1 - s)) * d + c0 : 0);
    }
    constexpr int kGroup = ONE ? 1 : (BR == 1 ? 8 : (BR == 2 ? 4 : 2));
    f32x4_t vv[kGroup];
    Raw4<BF16> hv[kGroup][BR];
    auto load_group = [&](int tg) {
        const int n = min(kGroup, t1 - tg);
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
            const int64_t row = row0 + tg + min(q, n - 1);
            vv[q] = *reinterpret_cast<const f32x4_t *>(a.v + row * d + cc0);
#pragma unroll
            for (int m = 0; m < BR; ++m) hv[q][m].load(a.h, ((int64_t)m * n_tok + row) * d + cc0);
        }
    };
    load_group(t0);
    float wt[4][kVec];
    load_taps<TAP4>(a.conv_w, kc, cc0, wt);

    for (int w = tid; w < n_sum; w += blockDim.x) sums_s[0][w] = sums_s[1][w] = sums_s[2][w] = 0.f;
    for (int q0 = 0; q0 < a.n_parts; q0 += q_round) {
        const int qn = min(q_round, a.n_parts - q0);
        // (the early values go to LDS on a path with no load of its own, so
        // their wait covers them alone)
        int x0 = tid;
        if (q0 == 0) {
#pragma unroll
            for (int i = 0; i < kPre; ++i)
                if (tid + i * (int)blockDim.x < qn * per_part) part_s[tid + i * blockDim.x] = pre[i];
            x0 = tid + kPre * blockDim.x;
        }
        for (int x = x0; x < qn * per_part; x += blockDim.x) part_s[x] = a.partials[part_at(x, q0)];
        __syncthreads();
        for (int w = tid; w < n_sum; w += blockDim.x) {
            const int m = w / npos, pi = w - m * npos;
            float s_hk = sums_s[0][w], s_kk = sums_s[1][w], s_hh = sums_s[2][w];
            for (int qq = 0; qq < qn; ++qq) {
                const int base = ((qq * BR + m) * 3) * npos + pi;
                s_hk += part_s[base];
                s_kk += part_s[base + npos];
                s_hh += part_s[base + 2 * npos];
            }
            sums_s[0][w] = s_hk;
            sums_s[1][w] = s_kk;
            sums_s[2][w] = s_hh;
        }
        __syncthreads();
    }
    // alpha_s[m][j] is the gate of position t0 - 3 + j (zero where unused)
    if constexpr (ONE) {
        // only alpha_s[m][3] is read.  No loop: for a loop that holds a
        // global store the compiler waits for every outstanding load before
        // entering it, the bulk loads above included (measured at a
        // 256-sequence decode step, four branches: 14.8 -> 14.2 us with this
        // and the straight-line position below)
        if (tid < BR) {
            const int m = tid;
            const float al = gate_finish(sums_s[0][m], sums_s[1][m], sums_s[2][m], d, a.eps);
            if (a.alpha && blockIdx.z == 0) a.alpha[m * n_tok + row0 + t0] = al;
            alpha_s[m][3] = al;
        }
    } else {
        for (int x = tid; x < BR * (kPos + 3); x += blockDim.x) {
            const int m = x / (kPos + 3), j = x - m * (kPos + 3);
            const int p = t0 - 3 + j;
            float al = 0.f;
            if (p >= pa && p < t1) {
                const int w = m * npos + (p - pa);
                al = gate_finish(sums_s[0][w], sums_s[1][w], sums_s[2][w], d, a.eps);
                if (a.alpha && p >= t0 && blockIdx.z == 0) a.alpha[m * n_tok + row0 + p] = al;
            }
            alpha_s[m][j] = al;
        }
    }
    __syncthreads();
    if (!live) return;

    const bool silu = a.conv_mode == ENGRAM_CONV_SILU_SKIP;
    const bool delta = (a.flags & ENGRAM_OUT_DELTA) != 0;

#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < kVec; ++c) wt[j][c] = j < kc ? wt[j][c] : 0.f;

    // win[m][s-1][c] = u_{t-s}
    float win[BR][3][kVec];
#pragma unroll
    for (int m = 0; m < BR; ++m)
#pragma unroll
        for (int s = 1; s <= 3; ++s) {
            const bool from_v = t0 - s >= 0;
            const float al = ONE ? 0.f : alpha_s[m][3 - s];  // (ONE: from_v is false)
#pragma unroll
            for (int c = 0; c < kVec; ++c) {
                const float vp = vprev_ok[s - 1] ? vprev[s - 1][c] : 0.f;
                const float sp = sprev_ok[s - 1] ? sprev[m][s - 1].get(c) : 0.f;
                win[m][s - 1][c] = from_v ? al * vp : sp;
            }
        }

    // position tg + q of the group in vv[q] / hv[q]
    auto position = [&](int tg, int q) {
        const int64_t row = row0 + tg + q;
#pragma unroll
        for (int m = 0; m < BR; ++m) {
            const float al = alpha_s[m][tg + q - t0 + 3];
            float o[kVec];
#pragma unroll
            for (int c = 0; c < kVec; ++c) {
                const float u = al * vv[q][c];
                const float conv = wt[0][c] * u + wt[1][c] * win[m][0][c] + wt[2][c] * win[m][1][c] +
                                   wt[3][c] * win[m][2][c];
                const float y = silu ? u + conv * sigmoidf_(conv) : conv;
                o[c] = delta ? y : hv[q][m].get(c) + y;
                win[m][2][c] = win[m][1][c];
                win[m][1][c] = win[m][0][c];
                win[m][0][c] = u;
            }
            Raw4<BF16>::store(a.out, ((int64_t)m * n_tok + row) * d + c0, o);
        }
    };
    if constexpr (ONE) {
        // straight-line code: in the loop below the next group's loads make
        // the compiler's waits at the loop head cover more than this position
        position(t0, 0);
    } else {
        for (int tg = t0; tg < t1; tg += kGroup) {
            const int n = min(kGroup, t1 - tg);
#pragma unroll
            for (int q = 0; q < kGroup; ++q) {
                if (q >= n) break;
                position(tg, q);
            }
            if (tg + kGroup < t1) load_group(tg + kGroup);
        }
    }

    // new conv state: the last K_c-1 gated values of the extended sequence
    if (a.state_stage && t1 == a.seqlen) {
#pragma unroll
        for (int m = 0; m < BR; ++m) {
            for (int j = 0; j < kc - 1; ++j) {
                const int64_t off = (((int64_t)m * a.batch + b) * (kc - 1) + j) * d + c0;
                const int s = kc - 1 - j;  // u_{T-s}
                float u4[kVec];
#pragma unroll
                for (int c = 0; c < kVec; ++c) u4[c] = s == 1 ? win[m][0][c] : (s == 2 ? win[m][1][c] : win[m][2][c]);
                if (a.stage_bf16)
                    *reinterpret_cast<u32x2_t *>(reinterpret_cast<uint16_t *>(a.state_stage) + off) =
                        u32x2_t{pack_bf16x2(u4[0], u4[1]), pack_bf16x2(u4[2], u4[3])};
                else
                    *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(a.state_stage) + off) =
                        f32x4_t{u4[0], u4[1], u4[2], u4[3]};
            }
        }
    }
}

}  // namespace

// One thread per (tile seam, 4 channels): the seam's three rows, every
// branch.  Tile T > 0, row rho < 3 (token t = 256 T + rho) belongs here when
// its sequence started before the tile (position > rho): u_{t-s} for s > rho
// then comes from the previous tile's last rows.  The six v rows around the
// seam (the previous tile's last three, this tile's first three), the taps
// and the six gates per branch are requested once for all three rows, before
// any arithmetic.  Same expressions, in the same order, as the projection
// kernel's epilogue, so the bits match the unsplit computation.
template <int BR, bool SILU>
__global__ __launch_bounds__(256) void seam_kernel(SeamArgs a) {
    const int d = a.d;
    const int quads = d / 4;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (int64_t)(a.n_tiles - 1) * quads) return;
    const int c0 = 4 * (int)(x % quads);
    const int T = 1 + (int)(x / quads);
    const int64_t tb = (int64_t)T * kTokTile;  // the tile's first token
    if (tb >= a.n_tok) return;
    const int kc = a.conv_k;
    const int64_t n_tok = a.n_tok;

    // vr[k + 3] = v of token tb + k, k = -3 .. 2: rows 3..5 of the previous
    // tile's seam rows, then rows 0..2 of this tile's (tokens past the end:
    // any valid row, never used)
    f32x4_t vr[6];
#pragma unroll
    for (int k = -3; k < 3; ++k) {
        const int64_t row = k >= 0 ? (int64_t)T * 6 + k : (int64_t)(T - 1) * 6 + 6 + k;
        vr[k + 3] = *reinterpret_cast<const f32x4_t *>(a.seam_v + row * d + c0);
    }
    f32x4_t tap[4];  // tap[r][s] multiplies u_{t-s} of channel c0 + r
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float w = a.conv_w[(int64_t)(c0 + r) * kc + max(kc - 1 - s, 0)];
            tap[r][s] = s < kc ? w : 0.f;
        }
    float al[BR][6];     // al[m][k + 3]: gate of token tb + k
    u32x2_t h2[BR][3];   // h of rows 0..2
#pragma unroll
    for (int m = 0; m < BR; ++m) {
#pragma unroll
        for (int k = -3; k < 3; ++k) al[m][k + 3] = a.alpha[m * n_tok + min(tb + k, n_tok - 1)];
#pragma unroll
        for (int rho = 0; rho < 3; ++rho)
            h2[m][rho] = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(a.h) +
                                                            ((int64_t)m * n_tok + min(tb + rho, n_tok - 1)) * d + c0);
    }
    const bool delta = (a.flags & ENGRAM_OUT_DELTA) != 0;

#pragma unroll
    for (int rho = 0; rho < 3; ++rho) {
        const int64_t t = tb + rho;
        if (t >= n_tok) break;
        const int b = (int)(t / a.seqlen);
        const int pos = (int)(t - (int64_t)b * a.seqlen);
        if (pos <= rho) continue;  // the projection kernel finished this row
#pragma unroll
        for (int m = 0; m < BR; ++m) {
            float u[4][4];  // u[s][r] = u_{t-s} of channel c0 + r
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (pos - s >= 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) u[s][r] = al[m][rho - s + 3] * vr[rho - s + 3][r];
                } else if (a.conv_state && s <= kc - 1) {
                    const f32x4_t st = load_state4(a.conv_state, a.state_bf16 != 0,
                                                   (((int64_t)m * a.batch + b) * (kc - 1) + (kc - 1) + pos - s) * d + c0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) u[s][r] = st[r];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) u[s][r] = 0.f;
                }
            }
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float conv = tap[r][0] * u[0][r] + tap[r][1] * u[1][r] + tap[r][2] * u[2][r] + tap[r][3] * u[3][r];
                const float y = SILU ? u[0][r] + conv * sigmoidf_(conv) : conv;
                const uint32_t hw = h2[m][rho][r >> 1];
                const float hval = bf16_to_f32((r & 1) ? (hw >> 16) : (hw & 0xFFFFu));
                o[r] = delta ? y : hval + y;
            }
            *reinterpret_cast<u32x2_t *>(reinterpret_cast<uint16_t *>(a.out) + ((int64_t)m * n_tok + t) * d + c0) =
                u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
    }
}

void launch_seam(const SeamArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)(a.n_tiles - 1) * (a.d / 4);
    if (items <= 0) return;
    const dim3 grid((unsigned)((items + 255) / 256));
    const bool silu = a.conv_mode == ENGRAM_CONV_SILU_SKIP;
#define ENGRAM_SEAM_LAUNCH(BR)                                                                    \
    do {                                                                                          \
        if (silu)                                                                                 \
            launch_kernel((seam_kernel<BR, true>), grid, dim3(256), s, a);                 \
        else                                                                                      \
            launch_kernel((seam_kernel<BR, false>), grid, dim3(256), s, a);                \
    } while (0)
    switch (a.n_branches) {
        case 1: ENGRAM_SEAM_LAUNCH(1); break;
        case 2: ENGRAM_SEAM_LAUNCH(2); break;
        case 3: ENGRAM_SEAM_LAUNCH(3); break;
        default: ENGRAM_SEAM_LAUNCH(4); break;
    }
#undef ENGRAM_SEAM_LAUNCH
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const f32x4_t *src, f32x4_t *dst, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const f32x4_t *src, u32x2_t *dst, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const f32x4_t x = src[i];
        dst[i] = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    }
}

void launch_f32_to_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t s) {
    const int64_t n4 = n / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    launch_kernel(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), s, reinterpret_cast<const f32x4_t *>(src),
                  reinterpret_cast<u32x2_t *>(dst), n4);
}

void launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t s) {
    const int64_t n4 = n / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    launch_kernel(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), s, reinterpret_cast<const f32x4_t *>(src),
                  reinterpret_cast<f32x4_t *>(dst), n4);
}

void launch_gate(const GateArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)((a.n_tok + 255) / 256), (unsigned)a.n_branches);
    launch_kernel(gate_kernel, grid, dim3(256), s, a);
}

void launch_fuse(const FuseArgs &a, engram_dtype dt, hipStream_t s) {
    const int need = (a.d + kVec - 1) / kVec;
    const int gz = (need + kFuseMaxThreads - 1) / kFuseMaxThreads;
    const int threads = ((need + gz - 1) / gz + 63) / 64 * 64;
    const dim3 grid((a.seqlen + kPos - 1) / kPos, a.batch, gz);
    const bool tap4 = a.conv_k == 4 && (reinterpret_cast<uintptr_t>(a.conv_w) & 15) == 0;
    const bool one = a.seqlen == 1;
    // (an fp32 plan carries an fp32 state)
#define ENGRAM_FUSE_SHAPE(BF, BR, SBF)                                                           \
    do {                                                                                         \
        if (one && tap4)                                                                         \
            launch_kernel((fuse_kernel<BF, BR, SBF, true, true>), grid, dim3(threads), s, a);    \
        else if (one)                                                                            \
            launch_kernel((fuse_kernel<BF, BR, SBF, false, true>), grid, dim3(threads), s, a);   \
        else if (tap4)                                                                           \
            launch_kernel((fuse_kernel<BF, BR, SBF, true, false>), grid, dim3(threads), s, a);   \
        else                                                                                     \
            launch_kernel((fuse_kernel<BF, BR, SBF, false, false>), grid, dim3(threads), s, a);  \
    } while (0)
#define ENGRAM_FUSE_LAUNCH(BR)                                                                   \
    do {                                                                                         \
        if (dt != ENGRAM_BF16)                                                                   \
            ENGRAM_FUSE_SHAPE(false, BR, false);                                                 \
        else if (a.state_bf16)                                                                   \
            ENGRAM_FUSE_SHAPE(true, BR, true);                                                   \
        else                                                                                     \
            ENGRAM_FUSE_SHAPE(true, BR, false);                                                  \
    } while (0)
    switch (a.n_branches) {
        case 1: ENGRAM_FUSE_LAUNCH(1); break;
        case 2: ENGRAM_FUSE_LAUNCH(2); break;
        case 3: ENGRAM_FUSE_LAUNCH(3); break;
        default: ENGRAM_FUSE_LAUNCH(4); break;
    }
#undef ENGRAM_FUSE_LAUNCH
#undef ENGRAM_FUSE_SHAPE
}

}  // namespace engram
