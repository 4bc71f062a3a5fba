// fuse.hip -- the rest of Engram's fusion step on gfx950 ([club] 1.(2)
// 上下文感知的门控机制, last two bullets; [csdn] Engram 到底怎么工作的, third
// and fourth steps): the scalar gate per token and branch from the partial
// sums the projection kernel left behind, the gated value u = alpha * v, the
// short depthwise causal convolution and the residual into the hidden state.
//
// HBM-bound: it reads v (fp32) once, h once per branch and writes out once
// per branch.  A block owns kPos consecutive positions of one sequence and a
// stripe of channels; each thread owns 8 channels (one 16-byte bf16 vector)
// and walks the positions in order, keeping the last three gated values of
// every branch in registers, so no gated value is ever written to memory.
// The three values before the block's first position are recomputed from v
// (or taken from the carried conv state at the sequence start).
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kPos = 32;
constexpr int kVec = 8;

template <bool BF16>
struct Vec8 {
    static __device__ __forceinline__ void load(const void *base, int64_t off, float (&x)[kVec]) {
        if constexpr (BF16) {
            const u32x4_t p = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint16_t *>(base) + off);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = bf16_to_f32(p[i] & 0xFFFFu);
                x[2 * i + 1] = bf16_to_f32(p[i] >> 16);
            }
        } else {
            const f32x4_t *p = reinterpret_cast<const f32x4_t *>(reinterpret_cast<const float *>(base) + off);
            const f32x4_t lo = p[0], hi = p[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = lo[i];
                x[4 + i] = hi[i];
            }
        }
    }
    static __device__ __forceinline__ void store(void *base, int64_t off, const float (&x)[kVec]) {
        if constexpr (BF16) {
            u32x4_t p;
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
            *reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(base) + off) = p;
        } else {
            f32x4_t *p = reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(base) + off);
            p[0] = f32x4_t{x[0], x[1], x[2], x[3]};
            p[1] = f32x4_t{x[4], x[5], x[6], x[7]};
        }
    }
};

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

template <bool BF16>
__global__ __launch_bounds__(512) void fuse_kernel(FuseArgs a) {
    __shared__ float alpha_s[kMaxBranches][kPos + 3];
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kPos;
    const int t1 = min(t0 + kPos, a.seqlen);
    const int64_t n_tok = (int64_t)a.batch * a.seqlen;
    const int64_t row0 = (int64_t)b * a.seqlen;
    const int d = a.d;
    const float inv_d = 1.f / (float)d;
    const float inv_sqrt_d = rsqrtf((float)d);

    // gate values for positions t0-3 .. t1-1 (zero where unused)
    for (int x = threadIdx.x; x < a.n_branches * (kPos + 3); x += blockDim.x) {
        const int m = x / (kPos + 3), j = x - m * (kPos + 3);
        const int p = t0 - 3 + j;
        float al = 0.f;
        if (p >= 0 && p < t1) {
            const float *pp = a.partials + (int64_t)m * a.n_parts * 3 * n_tok + row0 + p;
            float s_hk = 0.f, s_kk = 0.f, s_hh = 0.f;
            for (int q = 0; q < a.n_parts; ++q) {  // fixed order: bit-reproducible
                s_hk += pp[(3 * q + 0) * n_tok];
                s_kk += pp[(3 * q + 1) * n_tok];
                s_hh += pp[(3 * q + 2) * n_tok];
            }
            const float rh = sqrtf(s_hh * inv_d + a.eps);
            const float rk = sqrtf(s_kk * inv_d + a.eps);
            al = sigmoidf_(s_hk / (rh * rk) * inv_sqrt_d);
            if (a.alpha && p >= t0 && blockIdx.z == 0) a.alpha[m * n_tok + row0 + p] = al;
        }
        alpha_s[m][j] = al;
    }
    __syncthreads();

    const int c0 = (blockIdx.z * blockDim.x + threadIdx.x) * kVec;
    if (c0 >= d) return;
    const int kc = a.conv_k;

    float wt[4][kVec];  // wt[j][c] multiplies u_{t-j}
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < kVec; ++c)
            wt[j][c] = j < kc ? a.conv_w[(int64_t)(c0 + c) * kc + (kc - 1 - j)] : 0.f;

    // win[m][s-1][c] = u_{t-s}
    float win[kMaxBranches][3][kVec];
#pragma unroll
    for (int m = 0; m < kMaxBranches; ++m) {
        if (m >= a.n_branches) break;
#pragma unroll
        for (int s = 1; s <= 3; ++s) {
            const int p = t0 - s;
            float vv[kVec];
            if (p >= 0) {
                Vec8<false>::load(a.v, (row0 + p) * d + c0, vv);
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

    for (int t = t0; t < t1; ++t) {
        const int64_t row = row0 + t;
        float vv[kVec];
        Vec8<false>::load(a.v, row * d + c0, vv);
#pragma unroll
        for (int m = 0; m < kMaxBranches; ++m) {
            if (m >= a.n_branches) break;
            const float al = alpha_s[m][t - t0 + 3];
            const int64_t off = ((int64_t)m * n_tok + row) * d + c0;
            float hv[kVec], o[kVec];
            Vec8<BF16>::load(a.h, off, hv);
#pragma unroll
            for (int c = 0; c < kVec; ++c) {
                const float u = al * vv[c];
                const float conv = wt[0][c] * u + wt[1][c] * win[m][0][c] + wt[2][c] * win[m][1][c] +
                                   wt[3][c] * win[m][2][c];
                const float y = a.conv_mode == ENGRAM_CONV_SILU_SKIP ? u + conv * sigmoidf_(conv) : conv;
                o[c] = (a.flags & ENGRAM_OUT_DELTA) ? y : hv[c] + y;
                win[m][2][c] = win[m][1][c];
                win[m][1][c] = win[m][0][c];
                win[m][0][c] = u;
            }
            Vec8<BF16>::store(a.out, off, o);
        }
    }

    // new conv state: the last K_c-1 gated values of the extended sequence
    if (a.state_stage && t1 == a.seqlen) {
#pragma unroll
        for (int m = 0; m < kMaxBranches; ++m) {
            if (m >= a.n_branches) break;
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

void launch_fuse(const FuseArgs &a, engram_dtype dt, hipStream_t s) {
    const int need = (a.d + kVec - 1) / kVec;
    int threads = ((need + 63) / 64) * 64;
    if (threads > 512) threads = 512;
    const int gz = (need + threads - 1) / threads;
    dim3 grid((a.seqlen + kPos - 1) / kPos, a.batch, gz);
    if (dt == ENGRAM_BF16)
        hipLaunchKernelGGL(fuse_kernel<true>, grid, dim3(threads), 0, s, a);
    else
        hipLaunchKernelGGL(fuse_kernel<false>, grid, dim3(threads), 0, s, a);
}

}  // namespace engram
