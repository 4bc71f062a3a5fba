// proj_bf16.hip -- the dense contractions of Engram's fusion step on gfx950
// MFMA: k^(m) = W_k^(m) e and v = W_v e for every token ([club] 1.(2): the
// hidden state is the query, the retrieved embedding is key and value through
// projection matrices; [club] 2. 工程优化: branches share W_v, each has its
// own W_k).  One launch covers every projection: the weight rows of all
// W_k^(m) followed by W_v form the N dimension.
//
// Roles: the MFMA A operand is a tile of weight rows (n) and the B operand a
// tile of tokens (t), both K-contiguous ([d][D_e] weights, [n_tok][D_e] E), so
// each lane of a v_mfma_f32_16x16x32_bf16 result holds four consecutive
// output channels of one token.  That layout lets the gate epilogue reduce
// over channels mostly inside a lane:
//   W_k tiles never store k; they store per-token partial sums over their
//     128 channels of  h*gamma_h*gamma_k*k,  k^2  and  h^2  (the RMSNorm dot
//     product decomposes into these three sums).
//   W_v tiles store v (bf16) for the fusion kernel.
//
// Tile: 256 weight rows x 128 tokens x 64 K per stage, 4 waves as 2 x 2, each
// wave 128 x 64 (8 x 4 MFMA blocks, 128 fp32 accumulators per lane).  Both
// operand tiles are staged through LDS (rows padded by 16 bytes so the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks), double
// buffered with the next stage's global loads held in registers.
#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int BN = 256;           // weight rows per block
constexpr int BT = 128;           // tokens per block
constexpr int BK = 64;            // K per stage
constexpr int LDK = BK + 8;       // padded LDS row (bf16 elements)
constexpr int kThreads = 256;
constexpr int WN = 128, WT = 64;  // wave tile
constexpr int FN = WN / 16, FT = WT / 16;
constexpr int kLoadsW = BN * (BK / 8) / kThreads;  // 16-byte chunks per thread per stage
constexpr int kLoadsE = BT * (BK / 8) / kThreads;
constexpr int kXcds = 8;
constexpr int kGroupT = 4;        // token tiles interleaved per weight tile in the launch order

struct __attribute__((aligned(16))) Smem {
    uint16_t w[2][BN * LDK];
    uint16_t e[2][BT * LDK];
};

// Hardware hands consecutive block ids to the 8 XCDs round-robin.  Remap so
// every XCD walks one contiguous range of the logical tile order (its own
// L2 then sees neighbouring tiles), then order tiles in groups of kGroupT
// token tiles sharing each weight tile.
__device__ __forceinline__ void tile_of(int bid, int nblocks, int n_tiles_n, int n_tiles_t,
                                        int &tile_n, int &tile_t) {
    const int q = nblocks / kXcds, r = nblocks % kXcds;
    const int x = bid % kXcds, slot = bid / kXcds;
    const int logical = (x < r) ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
    const int per_group = kGroupT * n_tiles_n;
    const int g = logical / per_group;
    const int in = logical - g * per_group;
    const int t_base = g * kGroupT;
    const int gt = min(kGroupT, n_tiles_t - t_base);
    tile_n = in / gt;
    tile_t = t_base + (in - (in / gt) * gt);
}

// Select a[i] with constant indices only: a runtime index into a kernel
// argument array would make the compiler copy the arguments to memory.
template <typename T, int N>
__device__ __forceinline__ T pick(const T (&arr)[N], int i) {
    T p = arr[0];
#pragma unroll
    for (int j = 1; j < N; ++j)
        if (i == j) p = arr[j];
    return p;
}

__global__ __launch_bounds__(kThreads, 1) void proj_bf16_kernel(ProjArgs a) {
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int K = a.K;
    const int d = a.d;
    const int n_total = (a.n_branches + 1) * d;
    const int n_tiles_n = (n_total + BN - 1) / BN;
    const int n_tiles_t = (int)((a.n_tok + BT - 1) / BT);
    int tile_n, tile_t;
    tile_of(blockIdx.x, gridDim.x, n_tiles_n, n_tiles_t, tile_n, tile_t);
    const int n0 = tile_n * BN;
    const int64_t t0 = (int64_t)tile_t * BT;

    // ---- per-thread global source rows (fixed over the K loop).  Rows past
    //      the end are clamped to the last valid row: their products only
    //      reach outputs that are never written (n_total and the token count
    //      are checked in the epilogue), so no load ever leaves the buffers.
    const uint16_t *wsrc[kLoadsW];
    const uint16_t *esrc[kLoadsE];
    const int kc = (tid & 7) * 8;  // K offset of this thread's chunk within a stage
#pragma unroll
    for (int i = 0; i < kLoadsW; ++i) {
        const int n = min(n0 + (tid >> 3) + 32 * i, n_total - 1);
        const int mat = n / d;
        wsrc[i] = reinterpret_cast<const uint16_t *>(pick(a.w, mat)) + (int64_t)(n - mat * d) * K + kc;
    }
#pragma unroll
    for (int i = 0; i < kLoadsE; ++i) {
        const int64_t t = min(t0 + (tid >> 3) + 32 * i, a.n_tok - 1);
        esrc[i] = reinterpret_cast<const uint16_t *>(a.emb) + t * K + kc;
    }

    u32x4_t rw[kLoadsW], re[kLoadsE];
#define ENGRAM_LOAD_STAGE(k0)                                                                  \
    do {                                                                                       \
        _Pragma("unroll") for (int i = 0; i < kLoadsW; ++i)                                    \
            rw[i] = *reinterpret_cast<const u32x4_t *>(wsrc[i] + (k0));                          \
        _Pragma("unroll") for (int i = 0; i < kLoadsE; ++i)                                    \
            re[i] = *reinterpret_cast<const u32x4_t *>(esrc[i] + (k0));                          \
    } while (0)
#define ENGRAM_STORE_STAGE(buf)                                                                \
    do {                                                                                       \
        _Pragma("unroll") for (int i = 0; i < kLoadsW; ++i)                                    \
            *reinterpret_cast<u32x4_t *>(&sm.w[buf][((tid >> 3) + 32 * i) * LDK + kc]) = rw[i];  \
        _Pragma("unroll") for (int i = 0; i < kLoadsE; ++i)                                    \
            *reinterpret_cast<u32x4_t *>(&sm.e[buf][((tid >> 3) + 32 * i) * LDK + kc]) = re[i];  \
    } while (0)

    f32x4_t acc[FN][FT];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int wn = (wave & 1) * WN;   // wave's weight-row offset in the tile
    const int wt = (wave >> 1) * WT;  // wave's token offset in the tile
    const int frag_row = lane & 15;
    const int frag_k = (lane >> 4) * 8;

    const int k_steps = K / BK;
    ENGRAM_LOAD_STAGE(0);
    ENGRAM_STORE_STAGE(0);
    __syncthreads();
    for (int ks = 0; ks < k_steps; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < k_steps) ENGRAM_LOAD_STAGE((ks + 1) * BK);
        const uint16_t *lw = sm.w[buf];
        const uint16_t *le = sm.e[buf];
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8_t fa[FN], fb[FT];
#pragma unroll
            for (int i = 0; i < FN; ++i)
                fa[i] = *reinterpret_cast<const bf16x8_t *>(&lw[(wn + 16 * i + frag_row) * LDK + kk + frag_k]);
#pragma unroll
            for (int j = 0; j < FT; ++j)
                fb[j] = *reinterpret_cast<const bf16x8_t *>(&le[(wt + 16 * j + frag_row) * LDK + kk + frag_k]);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < k_steps) ENGRAM_STORE_STAGE(buf ^ 1);
        __syncthreads();
    }

#undef ENGRAM_LOAD_STAGE
#undef ENGRAM_STORE_STAGE

    // ---- epilogue.  acc[i][j][r] is output channel n = nw + 16i + 4*(lane/16) + r
    //      of token t = t0 + wt + 16j + lane%16.
    const int nw = n0 + wn;
    if (nw >= n_total) return;
    const int mat = nw / d;              // the wave's 128 rows lie in one matrix (d % 128 == 0)
    const int nl = nw - mat * d;         // first channel within that matrix
    const int sub = 4 * (lane >> 4);

    if (mat < a.n_branches) {
        // gate partials of branch `mat` over channels [nl, nl+128)
        const float *gh = pick(a.gamma_h, mat);
        const float *gk = pick(a.gamma_k, mat);
        float g[FN][4];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const float4 x = *reinterpret_cast<const float4 *>(gh + nl + 16 * i + sub);
            const float4 y = *reinterpret_cast<const float4 *>(gk + nl + 16 * i + sub);
            g[i][0] = x.x * y.x; g[i][1] = x.y * y.y; g[i][2] = x.z * y.z; g[i][3] = x.w * y.w;
        }
        const uint16_t *hm = reinterpret_cast<const uint16_t *>(a.h) + (int64_t)mat * a.n_tok * d;
        const int part = nl / kPartCols;
        float *pbase = a.partials + ((int64_t)mat * a.n_parts + part) * 3 * a.n_tok;
#pragma unroll
        for (int j = 0; j < FT; ++j) {
            const int64_t t = t0 + wt + 16 * j + (lane & 15);
            const bool live = t < a.n_tok;
            float s_hk = 0.f, s_kk = 0.f, s_hh = 0.f;
            const uint16_t *hrow = hm + (live ? t : 0) * d + nl + sub;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                uint2 hv = live ? *reinterpret_cast<const uint2 *>(hrow + 16 * i) : make_uint2(0, 0);
                const float h4[4] = {bf16_to_f32(hv.x & 0xFFFFu), bf16_to_f32(hv.x >> 16),
                                     bf16_to_f32(hv.y & 0xFFFFu), bf16_to_f32(hv.y >> 16)};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float kv = acc[i][j][r];
                    s_hk += h4[r] * g[i][r] * kv;
                    s_kk += kv * kv;
                    s_hh += h4[r] * h4[r];
                }
            }
            // the four lanes {l, l+16, l+32, l+48} hold the same token
            s_hk += __shfl_xor(s_hk, 16); s_hk += __shfl_xor(s_hk, 32);
            s_kk += __shfl_xor(s_kk, 16); s_kk += __shfl_xor(s_kk, 32);
            s_hh += __shfl_xor(s_hh, 16); s_hh += __shfl_xor(s_hh, 32);
            if (lane < 16 && live) {
                pbase[t] = s_hk;
                pbase[a.n_tok + t] = s_kk;
                pbase[2 * a.n_tok + t] = s_hh;
            }
        }
    } else {
        // v = W_v e, stored bf16 [n_tok][d]
        uint16_t *vout = reinterpret_cast<uint16_t *>(a.v);
#pragma unroll
        for (int j = 0; j < FT; ++j) {
            const int64_t t = t0 + wt + 16 * j + (lane & 15);
            if (t >= a.n_tok) continue;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                uint2 pk;
                pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *reinterpret_cast<uint2 *>(vout + t * d + nl + 16 * i + sub) = pk;
            }
        }
    }
}

}  // namespace

void launch_proj_bf16(const ProjArgs &a, hipStream_t s) {
    const int n_total = (a.n_branches + 1) * a.d;
    const int n_tiles_n = (n_total + BN - 1) / BN;
    const int64_t n_tiles_t = (a.n_tok + BT - 1) / BT;
    const int64_t blocks = (int64_t)n_tiles_n * n_tiles_t;
    hipLaunchKernelGGL(proj_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
}

}  // namespace engram
