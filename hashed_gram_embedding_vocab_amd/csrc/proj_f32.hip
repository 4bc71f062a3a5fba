// proj_f32.hip -- fp32 path of the fusion projections (tiny-configuration
// precision path): k^(m) = W_k^(m) e, v = W_v e in fp32 on the vector ALUs
// (MI355X's fp32 matrix and vector peaks are equal, so MFMA buys nothing
// here), followed by the per-token gate sums over all d channels.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int TN = 16, TT = 16, TK = 64;
constexpr int kOut = TN / 16;  // outputs per thread along n and along t
constexpr int kPer = TN * TK / 256;  // elements of each operand tile per thread and step

template <typename T, int N>
__device__ __forceinline__ T pick(const T (&arr)[N], int i) {
    T p = arr[0];
#pragma unroll
    for (int j = 1; j < N; ++j)
        if (i == j) p = arr[j];
    return p;
}

// C^T[n][t] = sum_k W[n][k] E[t][k] over the stacked rows of every W_k^(m)
// and W_v; k goes to kbuf[m][t][n'], v to v[t][n'].  Each step of TK columns
// requests all of its operand elements at once (every lane reads a valid
// element; out-of-range ones become zeros on their way into LDS), so a step
// costs one memory round trip; each output still adds k in order.
__global__ __launch_bounds__(256) void proj_f32_kernel(ProjArgs a) {
    __shared__ float ws[TN][TK + 1];
    __shared__ float es[TT][TK + 1];
    __shared__ const float *wmat_s[kMaxBranches + 1];  // the stacked matrices (a per-lane index into
                                                      // the kernel arguments would read them from memory)
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int d = a.d, K = a.K;
    const int n_total = (a.n_branches + 1) * d;
    const int n0 = blockIdx.x * TN;
    const int64_t t0 = (int64_t)blockIdx.y * TT;
    const float *emb = reinterpret_cast<const float *>(a.emb);
    float acc[kOut][kOut] = {};
    if (threadIdx.x <= kMaxBranches) wmat_s[threadIdx.x] = reinterpret_cast<const float *>(pick(a.w, threadIdx.x));
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += TK) {
        float wv[kPer], ev[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int x = threadIdx.x + 256 * u;
            const int r = x / TK, c = x % TK;
            const int n = min(n0 + r, n_total - 1), k = min(k0 + c, K - 1);
            const int mat = n / d;
            wv[u] = wmat_s[mat][(int64_t)(n - mat * d) * K + k];
            ev[u] = emb[min(t0 + r, a.n_tok - 1) * K + k];
        }
        asm volatile("" ::: "memory");  // every load above is issued before any goes to LDS
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int x = threadIdx.x + 256 * u;
            const int r = x / TK, c = x % TK;
            const bool kin = k0 + c < K;
            ws[r][c] = (n0 + r < n_total && kin) ? wv[u] : 0.f;
            es[r][c] = (t0 + r < a.n_tok && kin) ? ev[u] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk)
#pragma unroll
            for (int i = 0; i < kOut; ++i)
#pragma unroll
                for (int j = 0; j < kOut; ++j) acc[i][j] = fmaf(ws[tx + 16 * i][kk], es[ty + 16 * j][kk], acc[i][j]);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
        const int n = n0 + tx + 16 * i;
        if (n >= n_total) continue;
        const int mat = n / d, nl = n - mat * d;
#pragma unroll
        for (int j = 0; j < kOut; ++j) {
            const int64_t t = t0 + ty + 16 * j;
            if (t >= a.n_tok) continue;
            if (mat < a.n_branches)
                a.kbuf[((int64_t)mat * a.n_tok + t) * d + nl] = acc[i][j];
            else
                a.v[t * d + nl] = acc[i][j];
        }
    }
}

// Gate sums of one token and branch over all d channels (n_parts == 1).
__global__ __launch_bounds__(256) void gate_sums_f32_kernel(ProjArgs a) {
    __shared__ float red[3][256];
    const int64_t t = blockIdx.x;
    const int m = blockIdx.y;
    const int d = a.d;
    const float *k = a.kbuf + ((int64_t)m * a.n_tok + t) * d;
    const float *h = reinterpret_cast<const float *>(a.h) + ((int64_t)m * a.n_tok + t) * d;
    const float *gh = pick(a.gamma_h, m), *gk = pick(a.gamma_k, m);
    float s_hk = 0.f, s_kk = 0.f, s_hh = 0.f;
    for (int n = threadIdx.x; n < d; n += 256) {
        const float kv = k[n], hv = h[n];
        s_hk += hv * gh[n] * gk[n] * kv;
        s_kk += kv * kv;
        s_hh += hv * hv;
    }
    red[0][threadIdx.x] = s_hk;
    red[1][threadIdx.x] = s_kk;
    red[2][threadIdx.x] = s_hh;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w)
            for (int q = 0; q < 3; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x < 3) a.partials[((int64_t)m * 3 + threadIdx.x) * a.n_tok + t] = red[threadIdx.x][0];
}

}  // namespace

void launch_proj_f32(const ProjArgs &a, hipStream_t s) {
    const int n_total = (a.n_branches + 1) * a.d;
    dim3 grid((n_total + TN - 1) / TN, (unsigned)((a.n_tok + TT - 1) / TT));
    launch_kernel(proj_f32_kernel, grid, dim3(256), s, a);
    launch_kernel(gate_sums_f32_kernel, dim3((unsigned)a.n_tok, a.n_branches), dim3(256), s, a);
}

}  // namespace engram
