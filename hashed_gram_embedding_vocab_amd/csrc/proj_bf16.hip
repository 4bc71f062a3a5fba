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
//   W_v tiles store v (fp32) for the fusion kernel.
//
// Tile: 256 weight rows x 256 tokens (d % 256 == 0, so a weight tile never
// straddles two matrices), 32 K per stage (D_e % 128 == 0), 8 waves (two per
// SIMD) as 2 x 4, each wave 128 x 64 (8 x 4 MFMA blocks, 128 fp32
// accumulators per lane).  Operands go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds: no register staging, one 32-bit offset
// register per load, and reads past a buffer's end return zeros instead of
// faulting) through a ring of four 32 KB stages: while one stage is
// multiplied the next three are in flight, which covers the latency of
// operands that miss L2.  LDS holds each operand as 1 KB blocks of 16 rows x 32 K
// (one MFMA fragment); inside a block the four 16-byte chunks of a row are
// XOR-swizzled by ((r>>1) ^ (r>>2)) & 3 so the fragment reads of 8 or 16
// consecutive rows fall in distinct banks.
#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BN = 256;            // weight rows per block
constexpr int BT = 256;            // tokens per block
constexpr int BK = 32;             // K per stage (one MFMA K slab)
constexpr int kStages = 4;         // LDS ring: one stage multiplied, three in flight
constexpr int kThreads = 512;      // 8 waves: two per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int WN = 128, WT = 64;   // wave tile; waves form a 2 (n) x 4 (t) grid
constexpr int FN = WN / 16, FT = WT / 16;
constexpr int kBlockBytes = 1024;                       // 16 rows x 32 bf16
constexpr int kOperandBytes = (BN / 16) * kBlockBytes;  // 16 KB per operand per stage
constexpr int kBlocksPerWave = (BN / 16) / kWaves;          // row blocks each wave fills, per operand and stage
constexpr int kXcds = 8;
#ifndef ENGRAM_PROJ_GROUP_T
#define ENGRAM_PROJ_GROUP_T 4
#endif
constexpr int kGroupT = ENGRAM_PROJ_GROUP_T;  // token tiles sharing each weight tile in the launch order

static_assert(BN == BT, "one block-load pattern serves both operands");

struct __attribute__((aligned(1024))) Stage {
    unsigned char w[kOperandBytes];
    unsigned char e[kOperandBytes];
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

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

// Raw buffer resource over [base, base + bytes): dword 3 selects 32-bit data
// format with no swizzling, as every gfx9 raw buffer access expects.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence.  __syncthreads() would also
// wait for every outstanding load, including the next stage's LDS fills this
// kernel deliberately leaves in flight; visibility of a stage is instead
// established by each wave's own vmcnt wait before the barrier.  The empty
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kThreads, 1) void proj_bf16_kernel(ProjArgs a) {
    __shared__ Stage st0, st1, st2, st3;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
    const int K = a.K;
    const int d = a.d;
    const int n_total = (a.n_branches + 1) * d;
    const int n_tiles_n = (n_total + BN - 1) / BN;
    const int n_tiles_t = (int)((a.n_tok + BT - 1) / BT);
    int tile_n, tile_t;
    tile_of(blockIdx.x, gridDim.x, n_tiles_n, n_tiles_t, tile_n, tile_t);
    const int n0 = tile_n * BN;
    const int64_t t0 = (int64_t)tile_t * BT;

    // ---- this lane's share of the block loads.  Wave w fills row blocks
    //      2w and 2w+1 of each operand.
    //      Lane l fills row l>>2 of the block, LDS chunk l&3, which holds
    //      global K chunk (l&3) ^ swz(row).  Rows past the end are clamped to
    //      the last valid row: their products only reach outputs that the
    //      epilogue never writes, so no load leaves the buffers.
    const int lr = lane >> 2;
    const int lchunk = (lane & 3) ^ swz(lr);
    // d % 256 == 0, so a 256-row weight tile lies inside one matrix
    const int mat0 = min(n0, n_total - 1) / d;
    const char *wmat = reinterpret_cast<const char *>(pick(a.w, mat0));
    const __amdgpu_buffer_rsrc_t wres = make_rsrc(wmat, (uint32_t)d * K * 2u);
    const __amdgpu_buffer_rsrc_t eres = make_rsrc(a.emb, (uint32_t)(a.n_tok * K * 2));
    const int rows_left_t = (int)min<int64_t>(a.n_tok - t0, BT) - 1;  // last valid token row in the tile
    uint32_t woff[kBlocksPerWave], eoff[kBlocksPerWave];
#pragma unroll
    for (int i = 0; i < kBlocksPerWave; ++i) {
        const int row = (wave * kBlocksPerWave + i) * 16 + lr;
        woff[i] = (uint32_t)((n0 - mat0 * d + row) * K + lchunk * 8) * 2u;
        eoff[i] = (uint32_t)((t0 + min(row, rows_left_t)) * K + lchunk * 8) * 2u;
    }

// The immediate offset of a buffer load with an LDS destination moves the LDS
// address as well, so the K position travels in the scalar offset, which only
// moves the global address.
#define ENGRAM_ISSUE(STG, k0)                                                                    \
    do {                                                                                         \
        const int kbytes = (k0) * 2;                                                             \
        _Pragma("unroll") for (int i = 0; i < kBlocksPerWave; ++i) {                             \
            const int blk = wave * kBlocksPerWave + i;                                           \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t *)&STG.w[blk * kBlockBytes], \
                                                     16, woff[i], kbytes, 0, 0);                 \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(eres, (lds_void_t *)&STG.e[blk * kBlockBytes], \
                                                     16, eoff[i], kbytes, 0, 0);                 \
        }                                                                                        \
    } while (0)
    constexpr int kLoadsPerStage = 2 * kBlocksPerWave;  // per wave

    f32x4_t acc[FN][FT];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int wn_blk = (wave & 1) * (WN / 16);   // wave's first weight row block
    const int wt_blk = (wave >> 1) * (WT / 16);  // wave's first token row block (4 t-groups)
    const int fr = lane & 15;                    // fragment row
    const int fpos = fr * 64 + ((lane >> 4) ^ swz(fr)) * 16;  // byte offset inside a 1 KB block

#define ENGRAM_COMPUTE(STG)                                                                      \
    do {                                                                                         \
        bf16x8_t fa[FN], fb[FT];                                                                 \
        _Pragma("unroll") for (int i = 0; i < FN; ++i) fa[i] =                                   \
            *reinterpret_cast<const bf16x8_t *>(&STG.w[(wn_blk + i) * kBlockBytes + fpos]);      \
        _Pragma("unroll") for (int j = 0; j < FT; ++j) fb[j] =                                   \
            *reinterpret_cast<const bf16x8_t *>(&STG.e[(wt_blk + j) * kBlockBytes + fpos]);      \
        _Pragma("unroll") for (int i = 0; i < FN; ++i)                                           \
            _Pragma("unroll") for (int j = 0; j < FT; ++j)                                       \
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0); \
    } while (0)

    // Stage s lives in buffer s % 4 (D_e % 128 == 0, so the number of stages
    // is a multiple of four and the unrolled loop below names every buffer
    // statically).  Step s: wait until this wave's loads of stage s landed
    // (stages s+1 and s+2 may still be in flight), barrier (every wave's stage
    // s has landed, and every wave finished multiplying stage s-1), refill the
    // buffer of stage s-1 with stage s+3, multiply stage s.  The loop body has
    // no branches, so the compiler can tell which buffer each in-flight fill
    // targets and adds no waits of its own.
    const int k_steps = K / BK;
    ENGRAM_ISSUE(st0, 0 * BK);
    ENGRAM_ISSUE(st1, 1 * BK);
    ENGRAM_ISSUE(st2, 2 * BK);
    int ks = 0;
    for (; ks + 4 < k_steps; ks += 4) {  // every stage but the last four: s + 3 < k_steps
        wait_vmcnt<2 * kLoadsPerStage>();
        block_barrier();
        ENGRAM_ISSUE(st3, (ks + 3) * BK);
        ENGRAM_COMPUTE(st0);
        wait_vmcnt<2 * kLoadsPerStage>();
        block_barrier();
        ENGRAM_ISSUE(st0, (ks + 4) * BK);
        ENGRAM_COMPUTE(st1);
        wait_vmcnt<2 * kLoadsPerStage>();
        block_barrier();
        ENGRAM_ISSUE(st1, (ks + 5) * BK);
        ENGRAM_COMPUTE(st2);
        wait_vmcnt<2 * kLoadsPerStage>();
        block_barrier();
        ENGRAM_ISSUE(st2, (ks + 6) * BK);
        ENGRAM_COMPUTE(st3);
    }
    // the last four stages: ks = k_steps - 4; stages ks..ks+2 are in flight
    wait_vmcnt<2 * kLoadsPerStage>();
    block_barrier();
    ENGRAM_ISSUE(st3, (ks + 3) * BK);
    ENGRAM_COMPUTE(st0);
    wait_vmcnt<2 * kLoadsPerStage>();
    block_barrier();
    ENGRAM_COMPUTE(st1);
    wait_vmcnt<kLoadsPerStage>();
    block_barrier();
    ENGRAM_COMPUTE(st2);
    wait_vmcnt<0>();
    block_barrier();
    ENGRAM_COMPUTE(st3);
#undef ENGRAM_COMPUTE
#undef ENGRAM_ISSUE

    // ---- epilogue.  acc[i][j][r] is output channel n = nw + 16i + 4*(lane/16) + r
    //      of token t = tw + 16j + lane%16.
    const int nw = n0 + wn_blk * 16;
    if (nw >= n_total) return;
    const int mat = nw / d;       // the wave's 128 rows lie in one matrix (d % 128 == 0)
    const int nl = nw - mat * d;  // first channel within that matrix
    const int sub = 4 * (lane >> 4);
    const int64_t tw = t0 + wt_blk * 16;

    if (mat < a.n_branches) {
        // gate partials of branch `mat` over channels [nl, nl+128).
        // gamma_h * gamma_k for the wave's channels goes through the now idle
        // st0 (its last reader finished before the final barrier), so it costs
        // no registers; each wave writes and reads only its own 512 bytes.
        float *gsm = reinterpret_cast<float *>(st0.w) + wave * WN;
        {
            const float *gh = pick(a.gamma_h, mat);
            const float *gk = pick(a.gamma_k, mat);
            for (int c = lane; c < WN; c += 64) gsm[c] = gh[nl + c] * gk[nl + c];
        }
        const uint16_t *hm = reinterpret_cast<const uint16_t *>(a.h) + (int64_t)mat * a.n_tok * d;
        const int part = nl / kPartCols;
        float *pbase = a.partials + ((int64_t)mat * a.n_parts + part) * 3 * a.n_tok;
        // h for token block j+1 is in flight while block j is reduced
        u32x2_t hv[2][FN];
        auto load_h = [&](int j, u32x2_t(&dst)[FN]) {
            const int64_t t = min(tw + 16 * j + (lane & 15), a.n_tok - 1);
            const uint16_t *hrow = hm + t * d + nl + sub;
#pragma unroll
            for (int i = 0; i < FN; ++i) dst[i] = *reinterpret_cast<const u32x2_t *>(hrow + 16 * i);
        };
        load_h(0, hv[0]);
#pragma unroll
        for (int j = 0; j < FT; ++j) {
            if (j + 1 < FT) load_h(j + 1, hv[(j + 1) & 1]);
            const int64_t t = tw + 16 * j + (lane & 15);
            float s_hk = 0.f, s_kk = 0.f, s_hh = 0.f;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const u32x2_t x = hv[j & 1][i];
                const f32x4_t g = *reinterpret_cast<const f32x4_t *>(gsm + 16 * i + sub);
                const float h4[4] = {bf16_to_f32(x[0] & 0xFFFFu), bf16_to_f32(x[0] >> 16),
                                     bf16_to_f32(x[1] & 0xFFFFu), bf16_to_f32(x[1] >> 16)};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float kv = acc[i][j][r];
                    s_hk += h4[r] * g[r] * kv;
                    s_kk += kv * kv;
                    s_hh += h4[r] * h4[r];
                }
            }
            // the four lanes {l, l+16, l+32, l+48} hold the same token
            s_hk += __shfl_xor(s_hk, 16); s_hk += __shfl_xor(s_hk, 32);
            s_kk += __shfl_xor(s_kk, 16); s_kk += __shfl_xor(s_kk, 32);
            s_hh += __shfl_xor(s_hh, 16); s_hh += __shfl_xor(s_hh, 32);
            if (lane < 16 && t < a.n_tok) {
                pbase[t] = s_hk;
                pbase[a.n_tok + t] = s_kk;
                pbase[2 * a.n_tok + t] = s_hh;
            }
        }
    } else {
        // v = W_v e, kept fp32 [n_tok][d]: rounding it to bf16 here would add
        // up to half a bf16 ulp of |v| to every gated value the conv sums.
#pragma unroll
        for (int j = 0; j < FT; ++j) {
            const int64_t t = tw + 16 * j + (lane & 15);
            if (t >= a.n_tok) continue;
#pragma unroll
            for (int i = 0; i < FN; ++i)
                *reinterpret_cast<f32x4_t *>(a.v + t * d + nl + 16 * i + sub) = acc[i][j];
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
