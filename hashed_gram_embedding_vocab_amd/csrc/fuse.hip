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
// carried conv state at the sequence start).
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

// The gate of token t, branch m, from the n_parts partial sums, in a fixed
// order.  The one definition both kernels below use, so every path gets the
// same bits.
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
    const float inv_d = 1.f / (float)d;
    const float rh = sqrtf(s_hh * inv_d + eps);
    const float rk = sqrtf(s_kk * inv_d + eps);
    return sigmoidf_(s_hk / (rh * rk) * rsqrtf((float)d));
}

__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int m = blockIdx.y;
    if (a.ctx.prev_ctx && m == 0 && t < a.batch) ctx_update_one(a.ctx, (int32_t)t, a.seqlen);
    if (t >= a.n_tok) return;
    a.alpha[m * a.n_tok + t] = gate_value(a.partials, m, a.n_parts, a.n_tok, t, a.d, a.eps);
}

template <bool BF16, int BR>
__global__ __launch_bounds__(256) void fuse_kernel(FuseArgs a) {
    __shared__ float alpha_s[BR][kPos + 3];
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kPos;
    const int t1 = min(t0 + kPos, a.seqlen);
    const int64_t n_tok = (int64_t)a.batch * a.seqlen;
    const int64_t row0 = (int64_t)b * a.seqlen;
    const int d = a.d;

    if (a.ctx.prev_ctx && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) ctx_update_one(a.ctx, b, a.seqlen);
    // gate values for positions t0-3 .. t1-1 (zero where unused)
    for (int x = threadIdx.x; x < BR * (kPos + 3); x += blockDim.x) {
        const int m = x / (kPos + 3), j = x - m * (kPos + 3);
        const int p = t0 - 3 + j;
        float al = 0.f;
        if (p >= 0 && p < t1) {
            al = gate_value(a.partials, m, a.n_parts, n_tok, row0 + p, d, a.eps);
            if (a.alpha && p >= t0 && blockIdx.z == 0) a.alpha[m * n_tok + row0 + p] = al;
        }
        alpha_s[m][j] = al;
    }
    __syncthreads();

    const int c0 = (blockIdx.z * blockDim.x + threadIdx.x) * kVec;
    if (c0 >= d) return;
    const int kc = a.conv_k;
    const bool silu = a.conv_mode == ENGRAM_CONV_SILU_SKIP;
    const bool delta = (a.flags & ENGRAM_OUT_DELTA) != 0;

    float wt[4][kVec];  // wt[j][c] multiplies u_{t-j}
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < kVec; ++c)
            wt[j][c] = j < kc ? a.conv_w[(int64_t)(c0 + c) * kc + (kc - 1 - j)] : 0.f;

    // win[m][s-1][c] = u_{t-s}
    float win[BR][3][kVec];
#pragma unroll
    for (int m = 0; m < BR; ++m) {
#pragma unroll
        for (int s = 1; s <= 3; ++s) {
            const int p = t0 - s;
            if (p >= 0) {
                const f32x4_t vv = *reinterpret_cast<const f32x4_t *>(a.v + (row0 + p) * d + c0);
                const float al = alpha_s[m][3 - s];
#pragma unroll
                for (int c = 0; c < kVec; ++c) win[m][s - 1][c] = al * vv[c];
            } else if (a.conv_state && s <= kc - 1) {
                const float *st = a.conv_state + (((int64_t)m * a.batch + b) * (kc - 1) + (kc - 1 - s)) * d + c0;
#pragma unroll
                for (int c = 0; c < kVec; ++c) win[m][s - 1][c] = st[c];
            } else {
#pragma unroll
                for (int c = 0; c < kVec; ++c) win[m][s - 1][c] = 0.f;
            }
        }
    }

    constexpr int kGroup = BR == 1 ? 8 : (BR == 2 ? 4 : 2);
    for (int tg = t0; tg < t1; tg += kGroup) {
        const int n = min(kGroup, t1 - tg);
        f32x4_t vv[kGroup];
        Raw4<BF16> hv[kGroup][BR];
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
            const int64_t row = row0 + tg + min(q, n - 1);
            vv[q] = *reinterpret_cast<const f32x4_t *>(a.v + row * d + c0);
#pragma unroll
            for (int m = 0; m < BR; ++m) hv[q][m].load(a.h, ((int64_t)m * n_tok + row) * d + c0);
        }
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
            if (q >= n) break;
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
        }
    }

    // new conv state: the last K_c-1 gated values of the extended sequence
    if (a.state_stage && t1 == a.seqlen) {
#pragma unroll
        for (int m = 0; m < BR; ++m) {
            for (int j = 0; j < kc - 1; ++j) {
                float *st = a.state_stage + (((int64_t)m * a.batch + b) * (kc - 1) + j) * d + c0;
                const int s = kc - 1 - j;  // u_{T-s}
#pragma unroll
                for (int c = 0; c < kVec; ++c) st[c] = s == 1 ? win[m][0][c] : (s == 2 ? win[m][1][c] : win[m][2][c]);
            }
        }
    }
}

}  // namespace

// One thread per (seam row, 4 channels), branches in a loop.  Tile T > 0,
// row rho < 3 (token t = 256 T + rho) belongs here when its sequence started
// before the tile (position > rho): u_{t-s} for s > rho then comes from the
// previous tile's last rows.  Same expressions, in the same order, as the
// projection kernel's epilogue, so the bits match the unsplit computation.
template <int BR, bool SILU>
__global__ __launch_bounds__(256) void seam_kernel(SeamArgs a) {
    const int d = a.d;
    const int quads = d / 4;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (int64_t)(a.n_tiles - 1) * 3 * quads) return;
    const int c0 = 4 * (int)(x % quads);
    const int64_t rt = x / quads;
    const int rho = (int)(rt % 3);
    const int T = 1 + (int)(rt / 3);
    const int64_t t = (int64_t)T * kTokTile + rho;
    if (t >= a.n_tok) return;
    const int b = (int)(t / a.seqlen);
    const int pos = (int)(t - (int64_t)b * a.seqlen);
    if (pos <= rho) return;  // the projection kernel finished this row
    const int kc = a.conv_k;
    const int64_t n_tok = a.n_tok;

    // Every load below is issued unconditionally from an index that is
    // always valid (t - s >= 253 here), then selected: one memory round trip.
    // v of tokens t - s (s = 0..3): seam row rho - s of tile T, or row
    // 6 + rho - s of tile T-1 (its last three rows)
    f32x4_t vs[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int k = rho - s;
        const int64_t row = k >= 0 ? (int64_t)T * 6 + k : (int64_t)(T - 1) * 6 + 6 + k;
        vs[s] = *reinterpret_cast<const f32x4_t *>(a.seam_v + row * d + c0);
    }
    f32x4_t tap[4];  // tap[r][s] multiplies u_{t-s} of channel c0 + r
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float w = a.conv_w[(int64_t)(c0 + r) * kc + max(kc - 1 - s, 0)];
            tap[r][s] = s < kc ? w : 0.f;
        }
    const bool delta = (a.flags & ENGRAM_OUT_DELTA) != 0;
    float al[BR][4];
    u32x2_t h2[BR];
#pragma unroll
    for (int m = 0; m < BR; ++m) {
#pragma unroll
        for (int s = 0; s < 4; ++s) al[m][s] = a.alpha[m * n_tok + t - s];
        h2[m] = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(a.h) +
                                                   ((int64_t)m * n_tok + t) * d + c0);
    }

#pragma unroll
    for (int m = 0; m < BR; ++m) {
        float u[4][4];  // u[s][r] = u_{t-s} of channel c0 + r
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (pos - s >= 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) u[s][r] = al[m][s] * vs[s][r];
            } else if (a.conv_state && s <= kc - 1) {
                const float *st = a.conv_state + (((int64_t)m * a.batch + b) * (kc - 1) + (kc - 1) + pos - s) * d + c0;
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
            const uint32_t hw = h2[m][r >> 1];
            const float hval = bf16_to_f32((r & 1) ? (hw >> 16) : (hw & 0xFFFFu));
            o[r] = delta ? y : hval + y;
        }
        *reinterpret_cast<u32x2_t *>(reinterpret_cast<uint16_t *>(a.out) + ((int64_t)m * n_tok + t) * d + c0) =
            u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
}

void launch_seam(const SeamArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)(a.n_tiles - 1) * 3 * (a.d / 4);
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
    int threads = ((need + 63) / 64) * 64;
    if (threads > 256) threads = 256;
    const int gz = (need + threads - 1) / threads;
    dim3 grid((a.seqlen + kPos - 1) / kPos, a.batch, gz);
#define ENGRAM_FUSE_LAUNCH(BR)                                                                   \
    do {                                                                                         \
        if (dt == ENGRAM_BF16)                                                                   \
            launch_kernel((fuse_kernel<true, BR>), grid, dim3(threads), s, a);            \
        else                                                                                     \
            launch_kernel((fuse_kernel<false, BR>), grid, dim3(threads), s, a);           \
    } while (0)
    switch (a.n_branches) {
        case 1: ENGRAM_FUSE_LAUNCH(1); break;
        case 2: ENGRAM_FUSE_LAUNCH(2); break;
        case 3: ENGRAM_FUSE_LAUNCH(3); break;
        default: ENGRAM_FUSE_LAUNCH(4); break;
    }
#undef ENGRAM_FUSE_LAUNCH
}

}  // namespace engram
