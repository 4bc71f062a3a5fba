// proj_bf16.hip -- the dense contractions of Engram's fusion step on gfx950
// MFMA: k^(m) = W_k^(m) e and v = W_v e for every token ([club] 1.(2): the
// hidden state is the query, the retrieved embedding is key and value through
// projection matrices; [club] 2. 工程优化: branches share W_v, each has its
// own W_k).  Two modes share one main loop:
//   mode 0: the weight rows of the launch's matrices (all W_k^(m), optionally
//     followed by W_v) form the N dimension; W_k tiles leave gate partials,
//     W_v tiles store v.
//   mode 3: a plain contraction C[t][n] = sum_k W[n][k] E[t][k], fp32 out
//     (the backward's k, v and dE), optionally split over K.
//   mode 4: the same with both operands stored K-major (W^T and E^T, rows
//     of k): the backward's dW = [dk | dv]^T E contracts over tokens, and
//     both of its operands are token-major in memory.  The stages hold 32
//     k-rows of the tile's columns and the fragments come from transposing
//     LDS reads (ds_read_b64_tr_b16), so no operand is transposed in HBM.
//   mode 5: mode 3 over [W_k^(m); W_v] whose W_k tiles also leave mode 0's
//     gate partials (the backward's k and v, and its gate statistics).
//   mode 6: mode 3 whose weight side is read K-major from the stacked
//     matrices themselves (the backward's dE = [dk | dv] [W_k; W_v]: its
//     contraction runs over the matrices' rows), so W is not transposed.
//   mode 1: W_v only, with the rest of the fusion step in the epilogue:
//     alpha from the gate partials of a preceding mode-0 launch, u = alpha v,
//     the short depthwise causal conv over tokens, the residual into h and
//     the conv-state update ([club] 1.(2) last bullet).  v never reaches HBM.
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
// In mode 1 each lane holds four channels of one token per MFMA block and the
// 16 lanes of a row hold 16 consecutive tokens, so the conv's neighbours
// u_{t-1..t-3} come from DPP row rotations across lanes (plus the previous
// block's registers), and neighbouring waves of a tile pass three rows via
// LDS.  Token tiles do not overlap: each tile starts 256 tokens after the
// previous one, so the first three rows of a tile lack the previous tile's v.
// The tile leaves those rows, and saves the fp32 v of its first and last three
// rows, for seam_kernel (fuse.hip), which finishes them with the same
// expressions in the same order.
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
#include <type_traits>

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
constexpr int kHalo = 3;              // rows of conv history (K_c - 1 at most)
constexpr int kXcds = 8;
// Cache policy of the fused W_v epilogue's h loads and out stores: the "nt"
// (nontemporal) bit of the gfx950 buffer instructions.  That launch reads h for
// the last time and writes out, which this layer does not read again; streaming
// both past the caches keeps E and the weight tiles, which every workgroup of a
// token tile or channel tile rereads, resident.  Measured on the 200 GB tables
// (same bits): W_v 252 -> 228 us, and the next W_k 205 -> 194 us.  The W_k
// epilogue's h loads keep the default policy (W_v reads h again), and so do the
// operand loads (an E tile serves all d/256 channel tiles: nontemporal E loads
// made the W_v launch 1.4x slower).
constexpr int kCpolNT = 2;
#ifndef ENGRAM_PROJ_GROUP_T
#define ENGRAM_PROJ_GROUP_T 4
#endif
#ifndef ENGRAM_PROJ_GROUP_V
#define ENGRAM_PROJ_GROUP_V 1
#endif
// token tiles sharing each weight tile in the launch order: W_k and plain
// launches, and the fused W_v launch.  The W_v launch walks all channel tiles
// of one token tile before the next, so the workgroups of an XCD that run at
// once read and write whole token rows of h and out (measured against groups
// of four in alternating runs on one box: W_v 226 -> 218 us on the 200 GB
// tables, 0.462 -> 0.455 ms per step; W_k gains nothing from it).
constexpr int kGroupT = ENGRAM_PROJ_GROUP_T;
constexpr int kGroupV = ENGRAM_PROJ_GROUP_V;

static_assert(BN == BT, "one block-load pattern serves both operands");
static_assert(BT == kTokTile, "the seam kernel assumes this token tile");

// Tile shapes of proj_bf16_kernel: wide (256 x 256, 8 waves as 2 x 4) and
// narrow (128 x 128, 4 waves as 1 x 4).
template <bool NARROW>
struct TileCfg {
    static constexpr int BN = NARROW ? 128 : 256;                 // weight rows per block
    static constexpr int BT = NARROW ? 128 : 256;                 // tokens per block
    static constexpr int kThreads = NARROW ? 256 : 512;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kWavesN = NARROW ? 1 : 2;                // waves along n
    static constexpr int WT = BT / (kWaves / kWavesN);            // tokens per wave
    static constexpr int FT = WT / 16;
    static constexpr int kOperandBytes = (BN / 16) * kBlockBytes; // per operand and stage
    static constexpr int kBlocksPerWave = (BN / 16) / kWaves;     // row blocks each wave fills
    static_assert(BN == BT && kBlocksPerWave >= 1 && FN * 16 * kWavesN == BN, "tile shape");
};

template <int OPB>
struct __attribute__((aligned(1024))) StageT {
    unsigned char w[OPB];
    unsigned char e[OPB];
};
typedef StageT<kOperandBytes> Stage;

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Mode 4 stages: k-row kr of an operand is RB = 2 x (tile columns) bytes of
// LDS, 16-byte chunks; chunk pair q (columns 16q..16q+15) of row kr sits at
// pair position q ^ kswz(kr).  One transposing read covers 16 k-rows
// kr = 8g + 4h + r (g, r = 0..3) of one column block; kswz sends them to
// distinct pair positions (16 in a 512-byte row, 8 in a 256-byte one).
template <int PAIRS>
__device__ __forceinline__ int kswz(int kr) {
    return ((kr & 3) | (((kr >> 3) & 3) << 2)) & (PAIRS - 1);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4_t lds_read_tr(const unsigned char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t *)(const_cast<unsigned char *>(p)));
}

// Hardware hands consecutive block ids to the 8 XCDs round-robin.  Remap so
// every XCD walks one contiguous range of the logical tile order (its own
// L2 then sees neighbouring tiles), then order tiles in groups of G token
// tiles sharing each weight tile.
template <int G>
__device__ __forceinline__ void tile_of(int bid, int nblocks, int n_tiles_n, int n_tiles_t,
                                        int &tile_n, int &tile_t) {
    const int q = nblocks / kXcds, r = nblocks % kXcds;
    const int x = bid % kXcds, slot = bid / kXcds;
    const int logical = (x < r) ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
    const int per_group = G * n_tiles_n;
    const int g = logical / per_group;
    const int in = logical - g * per_group;
    const int t_base = g * G;
    const int gt = min(G, n_tiles_t - t_base);
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

// Workgroup barrier without a vector-memory wait.  __syncthreads() would
// also wait for every outstanding load, including the next stage's LDS fills
// this kernel deliberately leaves in flight; visibility of a stage is instead
// established by each wave's own vmcnt wait before the barrier.  The wave's
// own LDS reads are drained first (lgkmcnt(0)): the compiler may otherwise
// issue a stage's last fragment reads before the barrier and wait for them
// after it, and the buffer they read is refilled by DMA right after the
// barrier.  The empty asm statements keep the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// x from lane (l - s) of the same 16-lane row (rotating), s in 1..3
template <int S>
__device__ __forceinline__ float row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + S, 0xF, 0xF, false));
}

// s_waitcnt lgkmcnt(0) alone: every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// Byte offset (in one branch of h or out) of the 16-byte piece that lane
// moves with chunk instruction k of the mode-1 epilogue: LDS row p = 8k +
// lane/8 of the wave's 64 tokens (token t0 + rowbase + p, clamped into the
// tokens), piece lane%8 of the row, read from global piece (lane%8) ^ ((p/4) % 8).
__device__ __forceinline__ uint32_t chunk_offset(int k, int lane, int rowbase, int64_t t0, int64_t n_tok, int d,
                                                 int nl) {
    const int p = 8 * k + (lane >> 3);
    const int64_t tok = min(max(t0 + rowbase + p, (int64_t)0), n_tok - 1);
    return (uint32_t)((tok * d + nl) * 2) + (uint32_t)(((lane & 7) ^ ((p >> 2) & 7)) << 4);
}

// Mode-1 epilogue.  The tile's E rows were loaded so that in each wave's
// group of 64 tokens, lane row l (l = lane % 16) holds tokens 4l + j in its
// accumulator blocks j = 0..3: acc[i][j][r] is v of channel
// nl + 16i + 4*(lane/16) + r and token t0 + 64g + 4l + j.  For the conv,
// u_{t-s} then lies in the same lane (block j - s) when s <= j, else in lane
// row l - 1 (block j - s + 4, one DPP row shift), or for lane row 0 among the
// previous group's last three tokens, which pass through LDS.  The first
// group's first three rows need the previous tile's last three tokens unless a
// sequence starts close enough (position <= row); those rows are left to
// the seam kernel, which finishes them from the fp32 v of both tiles' edge
// rows that every block saves (seam_v).
//
// h arrives in LDS by DMA, one 8 KB chunk (64 tokens x 64 channels of one
// branch) per wave at a time, two chunks in flight, so the loads need no
// registers and overlap the arithmetic of the previous chunk.  Chunk c holds
// branch c/2, channels nl + 64(c%2) .. +63, in buffer hA (c even) or hB
// (c odd); LDS row p is token 64g + p, its eight 16-byte pieces XOR-swizzled
// by (p/4) % 8.  Each lane overwrites the h values it read with out, and the
// chunk goes back to memory the way it came, eight whole 128-byte rows per
// store.  Every store is issued (rows the tile must not write get an offset
// past the buffer, which the hardware drops), so the number of memory
// operations between two chunk loads is known and the waits below are exact.
template <int BR, bool SILU>
__device__ __forceinline__ void fused_value_epilogue(const ProjArgs &a, f32x4_t (&acc)[FN][FT],
                                                     float (&alpha_s)[BR][BT], float *halo, float *taps,
                                                     unsigned char *hA, unsigned char *hB, int wave,
                                                     int lane, int nl, int n0, int tile_t, int64_t t0) {
    const int d = a.d;
    const int l16 = lane & 15;
    const int sub = 4 * (lane >> 4);
    const int g = wave >> 1;
    const int rowbase = 64 * g;
    const int64_t n_tok = a.n_tok;
    const int kc = a.conv_k;
    const bool delta = (a.flags & ENGRAM_OUT_DELTA) != 0;

    // the block's 256 channels of conv taps, as taps[c][s] multiplying
    // u_{t-s} (zero beyond K_c)
    for (int x = threadIdx.x; x < BN; x += kThreads) {
        f32x4_t w4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < kc) w4[q] = a.conv_w[(int64_t)(n0 + x) * kc + (kc - 1 - q)];
        *reinterpret_cast<f32x4_t *>(&taps[4 * x]) = w4;
    }
    // the group's last three tokens (lane row 15, blocks 1..3) for the wave
    // holding the next 64 tokens of the same channels: halo row j-1 is token 60+j
    if (l16 == 15) {
#pragma unroll
        for (int j = 1; j < FT; ++j)
#pragma unroll
            for (int i = 0; i < FN; ++i)
                *reinterpret_cast<f32x4_t *>(&halo[(wave * kHalo + (j - 1)) * WN + 16 * i + sub]) = acc[i][j];
    }
    // v of the tile's first and last three rows, for the seam kernel (issued
    // before the chunk loads below, so they do not enter the waits there)
    // (seam row k of tile T is at seam_v[(6T + k) * d]: rows 0..2 are tile
    // rows 0..2, blocks 0..2 of lane row 0 of the first group; rows 3..5 are
    // tile rows BT-3..BT-1, blocks 1..3 of lane row 15 of the last group)
    float *sv = a.seam_v + (int64_t)tile_t * 6 * d + nl + sub;
    if (g == 0 && l16 == 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int i = 0; i < FN; ++i) *reinterpret_cast<f32x4_t *>(sv + (int64_t)j * d + 16 * i) = acc[i][j];
    }
    if (g == kWaves / 2 - 1 && l16 == 15) {
#pragma unroll
        for (int j = 1; j < FT; ++j)
#pragma unroll
            for (int i = 0; i < FN; ++i)
                *reinterpret_cast<f32x4_t *>(sv + (int64_t)(2 + j) * d + 16 * i) = acc[i][j];
    }
    __syncthreads();  // taps and halo written; every wave is done with the stage buffers
    // the first group's rows before its own take no values from a neighbour
    // (it reads its own halo rows, finite, times a zero gate: no branch)
    const bool has_prev = g > 0;
    const float *prev = halo + (has_prev ? wave - 2 : wave) * kHalo * WN;

    const uint32_t branch_bytes = (uint32_t)(n_tok * d * 2);
    const uint32_t state_branch_bytes = (uint32_t)a.batch * (uint32_t)(kc - 1) * (uint32_t)d * 4u;
    const uint32_t state_row_bytes = (uint32_t)d * 4u;
    const __amdgpu_buffer_rsrc_t hres = make_rsrc(a.h, branch_bytes * BR);
    const __amdgpu_buffer_rsrc_t ores = make_rsrc(a.out, branch_bytes * BR);
    // a bf16 state has every byte offset of the fp32 layout halved
    const bool state_bf16 = a.state_bf16 != 0;
    const __amdgpu_buffer_rsrc_t cres = make_rsrc(a.conv_state, (state_branch_bytes * BR) >> (state_bf16 ? 1 : 0));
    const __amdgpu_buffer_rsrc_t sres = make_rsrc(a.state_stage, state_branch_bytes * BR);
    // the new state's rows are the gated values of the last K_c-1 positions
    const uint32_t stage_shift = (uint32_t)(a.seqlen - (kc - 1)) * state_row_bytes;

    int pos[FT];
    bool edge[FT], to_state[FT];
    uint32_t srow[FT], stagerow[FT];
#pragma unroll
    for (int j = 0; j < FT; ++j) {
        const int row = rowbase + 4 * l16 + j;
        const int64_t tt = t0 + row;
        const bool valid = tt >= 0 && tt < n_tok;
        const int tc = valid ? (int)tt : 0;
        const int bseq = tc / a.seqlen;
        pos[j] = tc - bseq * a.seqlen;
        to_state[j] = valid && pos[j] >= a.seqlen - (kc - 1);
        // rows that need carried state (sequence start) or write it (sequence end)
        edge[j] = __ballot(valid && (pos[j] < kHalo || to_state[j])) != 0;
        // byte offset of state row pos of sequence bseq, modulo 2^32: exact
        // (in range) for the rows that read or write the state
        srow[j] = ((uint32_t)bseq * (uint32_t)(kc - 1) + (uint32_t)pos[j]) * state_row_bytes +
                  (uint32_t)(nl + sub) * 4u;
        stagerow[j] = srow[j] - stage_shift;
    }

    const bool any_edge = edge[0] || edge[1] || edge[2] || edge[3];
    const bool carry = a.conv_state != nullptr;

    // chunk DMA: instruction k fills LDS rows 8k .. 8k+7 (lane -> row
    // 8k + lane/8, piece lane%8), so lane reads global piece
    // (lane%8) ^ swizzle(row) of its token's 64 channels.  out goes back
    // the same way (same offsets), for the rows the tile writes: bit k of
    // store_rows.  Rows whose conv history reaches into the previous tile
    // are the seam kernel's (their state rows, plain gated values, are
    // written here).
    uint32_t hoff[8];
    uint32_t store_rows = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int p = 8 * k + (lane >> 3);
        const int row = rowbase + p;
        const int64_t tt = t0 + row;
        const int64_t tok = min(max(tt, (int64_t)0), n_tok - 1);
        hoff[k] = chunk_offset(k, lane, rowbase, t0, n_tok, d, nl);
        bool store = tt < n_tok;
        if (row < kHalo) store = store && (int)(tok % a.seqlen) <= row;
        if (store) store_rows |= 1u << k;
    }
    auto issue = [&](unsigned char *buf, int c) {
        wait_lgkm0();  // this wave's reads of the buffer's previous chunk are done
        asm volatile("" ::: "memory");
        const int soff = (int)(branch_bytes * (uint32_t)(c >> 1)) + 128 * (c & 1);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(hres, (lds_void_t *)(buf + k * 1024), 16, hoff[k], soff, 0,
                                                     kCpolNT);
    };
    // LDS byte offset of this lane's 4 channels of block i' of a chunk, token
    // row 4*l16 (+ 128 bytes per block j): piece 2i' + sub/8, swizzled by l16 % 8
    uint32_t ldo[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
        ldo[ii] = (uint32_t)(l16 * 512 + (((2 * ii + (sub >> 3)) ^ (l16 & 7)) << 4) + (sub & 4) * 2);

    // EDGE: some token block of the wave holds a sequence's first or last
    // positions.  Without it the body is straight-line code.  CARRY: a
    // carried conv state is read there (without one, the history before a
    // sequence start is zero and nothing is loaded or waited for: the wait
    // would otherwise drain the next chunk's h load and the last chunk's
    // stores in every wave holding a sequence edge).
    auto chunk = [&](auto qc, auto ec, auto cc, unsigned char *buf, int m, int moff, int smoff,
                     const float (&al)[FT], const float (&alh)[3]) {
        constexpr int q = decltype(qc)::value;
        constexpr bool EDGE = decltype(ec)::value;
        constexpr bool CARRY = decltype(cc)::value;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            asm volatile("" ::: "memory");  // one channel group at a time: bounds register use
            const int i = 4 * q + ii;
            const int c0 = nl + 16 * i + sub;
            f32x4_t tap[4];  // tap[r][s] multiplies u_{t-s} of channel c0 + r
#pragma unroll
            for (int r = 0; r < 4; ++r) tap[r] = *reinterpret_cast<const f32x4_t *>(&taps[4 * (c0 + r - n0)]);
            float u[FT][4];
#pragma unroll
            for (int j = 0; j < FT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) u[j][r] = al[j] * acc[i][j][r];
            // pr[s-1][r] = u_{4l-s}: block 4-s of lane row l-1; for lane row 0
            // the previous group's token 64-s (DPP row shift keeps `old` there)
            float pr[3][4];
#pragma unroll
            for (int s = 1; s <= 3; ++s) {
                const f32x4_t hp = *reinterpret_cast<const f32x4_t *>(&prev[(3 - s) * WN + 16 * i + sub]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    pr[s - 1][r] = __int_as_float(__builtin_amdgcn_update_dpp(
                        __float_as_int(alh[s - 1] * hp[r]), __float_as_int(u[4 - s][r]), 0x111, 0xF, 0xF, false));
            }
#pragma unroll
            for (int j = 0; j < FT; ++j) {
                f32x4_t sh[3];  // sh[s-1][r] = u_{t-s} of channel c0 + r
#pragma unroll
                for (int s = 1; s <= 3; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sh[s - 1][r] = j >= s ? u[j - s][r] : pr[s - j - 1][r];
                if (EDGE && edge[j]) {  // wave-uniform: a sequence starts or ends among these rows
                    // u before a sequence's first position is its carried state
                    // (state row K_c-1-s of the sequence for u_{-s}), or zero
                    // beyond it.  Lanes that do not need it read offset 0 of
                    // the branch's state, so every lane stays inside the buffer.
                    // (The empty asm makes sr opaque here, so the offsets
                    // derived from it are not hoisted out of the branch loop.)
                    uint32_t sr = srow[j];
                    asm volatile("" : "+v"(sr));
#pragma unroll
                    for (int s = 1; s <= 3; ++s) {
                        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
                        if (CARRY && s <= kc - 1) {
                            const uint32_t off = pos[j] < s ? sr + 64u * i : 0u;
                            const int soff = smoff + (kc - 1 - s) * (int)state_row_bytes;
                            if (state_bf16) {
                                const u32x2_t x = __builtin_bit_cast(
                                    u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(cres, off >> 1, soff >> 1, 0));
                                c = f32x4_t{bf16_to_f32(x[0] & 0xFFFFu), bf16_to_f32(x[0] >> 16),
                                            bf16_to_f32(x[1] & 0xFFFFu), bf16_to_f32(x[1] >> 16)};
                            } else {
                                c = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cres, off, soff, 0));
                            }
                        }
                        if (pos[j] < s) sh[s - 1] = c;
                    }
                    // drain here: left pending, the compiler would wait for
                    // them (and everything before) after the branch, on every path
                    if constexpr (CARRY) {
                        wait_vmcnt<0>();
                        asm volatile("" ::: "memory");
                    }
                }
                const u32x2_t h2 = *reinterpret_cast<const u32x2_t *>(buf + ldo[ii] + 128 * j);
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float conv =
                        tap[r][0] * u[j][r] + tap[r][1] * sh[0][r] + tap[r][2] * sh[1][r] + tap[r][3] * sh[2][r];
                    const float y = SILU ? u[j][r] + conv * sigmoid_f(conv) : conv;
                    const uint32_t hw = h2[r >> 1];
                    const float hval = bf16_to_f32((r & 1) ? (hw >> 16) : (hw & 0xFFFFu));
                    o[r] = delta ? y : hval + y;
                }
                // out replaces h in the chunk buffer (same place, same lane)
                *reinterpret_cast<u32x2_t *>(buf + ldo[ii] + 128 * j) =
                    u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                if (EDGE && edge[j] && a.state_stage && to_state[j])
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4_t, f32x4_t{u[j][0], u[j][1], u[j][2], u[j][3]}), sres,
                        stagerow[j] + 64 * i, smoff, 0);
            }
        }
        // out leaves in the layout h arrived in: each store writes eight whole
        // 128-byte rows (storing straight from the MFMA layout would write 16
        // rows x 32 bytes per instruction, a quarter line each).  Every store
        // is issued; rows the tile does not write go past the buffer's end.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(buf + k * 1024 + lane * 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, ores, ((store_rows >> k) & 1u) ? hoff[k] : 0x80000000u,
                                                   moff + 128 * q, kCpolNT);
        }
    };

    // Issue order: load(0) (by the main loop, into buffer A as soon as the
    // ring released it), load(1), chunk 0's 8 stores, load(2), chunk 1's
    // stores, load(3), ...  Before chunk c, the operations issued after
    // load(c) are chunk c-1's stores (8, for c >= 1) and load(c+1) (8, if
    // there is one).  Vector memory operations complete in issue order, so
    // waiting until no more than those are outstanding means chunk c has
    // landed.  State stores and carried-state loads near sequence edges, and
    // the seam rows stored above after load(0), only add operations, which
    // makes these waits stricter, never looser.
    issue(hB, 1);
#pragma unroll 1
    for (int m = 0; m < BR; ++m) {
        const int moff = (int)(branch_bytes * (uint32_t)m);
        const int smoff = (int)(state_branch_bytes * (uint32_t)m);
        float al[FT], alh[3];
#pragma unroll
        for (int j = 0; j < FT; ++j) al[j] = alpha_s[m][rowbase + 4 * l16 + j];
#pragma unroll
        for (int s = 1; s <= 3; ++s) alh[s - 1] = has_prev ? alpha_s[m][rowbase - s] : 0.f;
        if (m == 0)
            wait_vmcnt<8>();
        else
            wait_vmcnt<16>();
        asm volatile("" ::: "memory");
        if (any_edge && carry)
            chunk(std::integral_constant<int, 0>{}, std::true_type{}, std::true_type{}, hA, m, moff, smoff, al, alh);
        else if (any_edge)
            chunk(std::integral_constant<int, 0>{}, std::true_type{}, std::false_type{}, hA, m, moff, smoff, al, alh);
        else
            chunk(std::integral_constant<int, 0>{}, std::false_type{}, std::false_type{}, hA, m, moff, smoff, al, alh);
        if (m + 1 < BR) issue(hA, 2 * m + 2);
        if (m + 1 < BR)
            wait_vmcnt<16>();
        else
            wait_vmcnt<8>();
        asm volatile("" ::: "memory");
        if (any_edge && carry)
            chunk(std::integral_constant<int, 1>{}, std::true_type{}, std::true_type{}, hB, m, moff, smoff, al, alh);
        else if (any_edge)
            chunk(std::integral_constant<int, 1>{}, std::true_type{}, std::false_type{}, hB, m, moff, smoff, al, alh);
        else
            chunk(std::integral_constant<int, 1>{}, std::false_type{}, std::false_type{}, hB, m, moff, smoff, al, alh);
        if (m + 1 < BR) issue(hB, 2 * m + 3);
    }
}

// MODE 0, or MODE 1 with BR branches and the conv output passed through
// SiLU plus the skip term (SILU) or not.  MODE 2 is mode 0 (narrow tile only)
// with its E operand read from the tables: the block first hashes the
// n-grams of its 128 tokens into LDS, then each lane's 16-byte piece of a
// stage comes from the table row its token's slot names.  NARROW (modes 0, 2, 3): tiles of 128
// weight rows x 128 tokens and 4 waves of 128 x 32, for launches with too few
// 256 x 256 tiles to fill the chip (decode).  A wave always owns 128 output
// channels in the same MFMA layout, so the gate partial sums come out
// bit-identical whichever tile computed them.
template <int MODE, int BR, bool SILU, bool NARROW, bool TG = false>
__global__ __launch_bounds__(NARROW ? 256 : kThreads, NARROW ? 2 : 1) void proj_bf16_kernel(ProjArgs a) {
    static_assert(!(NARROW && MODE == 1), "the fused value epilogue is written for the wide tile");
    static_assert(!TG || (!NARROW && (MODE == 0 || MODE == 1)), "TG: wide W_k or W_v launch reading the tables");
    static_assert(MODE >= 0 && MODE <= 6, "mode");
    constexpr bool kKMajW = MODE == 4 || MODE == 6;  // weight-side operand stored K-major
    constexpr bool kKMajE = MODE == 4;               // token-side operand stored K-major
    constexpr bool kPlain = MODE == 3 || MODE == 4 || MODE == 5 || MODE == 6;  // fp32 store epilogue
    static_assert(MODE != 2 || NARROW, "retrieval inside the launch is written for the narrow tile");
    // retrieval inside the launch: the narrow mode 2, or a wide W_k / W_v launch with TG
    constexpr bool kGather = MODE == 2 || TG;
    constexpr bool kGateK = MODE == 0 || MODE == 2 || MODE == 5;  // W_k / W_v launch with the gate-partial epilogue
    typedef TileCfg<NARROW> C;
    constexpr int TBN = C::BN, TBT = C::BT, TTHREADS = C::kThreads, TWAVES = C::kWaves, TWGN = C::kWavesN;
    constexpr int TWT = C::WT, TFT = C::FT, TOPB = C::kOperandBytes, TBPW = C::kBlocksPerWave;
    __shared__ StageT<TOPB> st0, st1, st2, st3;
    __shared__ float alpha_s[MODE == 1 ? BR : 1][TBT];
    __shared__ __attribute__((aligned(16))) float gsm_s[kGateK ? TWAVES * WN : 4];
    // The W_v launch reading the tables keeps its slot table in the space of
    // the epilogue's taps and halo rows (LDS would not hold both): the slots
    // are read only while the ring is filled, the taps and halo rows written
    // only after the ring's last barrier.
    // (taps_own is then one buffer: the slots while the ring fills, the taps
    // and after them the halo rows in the epilogue)
    constexpr bool kSlotsInEpi = TG && MODE == 1;
    constexpr int kEpiFloats = 4 * TBN + TWAVES * kHalo * WN;
    constexpr int kSlots = TBT * kGatherMaxTables;
    __shared__ uint32_t idx_own[kGather && !kSlotsInEpi ? kSlots : 1];  // slot of (token of the tile, table)
    __shared__ const char *tab_s[kGather ? kGatherMaxTables : 1];
    __shared__ __attribute__((aligned(16)))
    float taps_own[MODE == 1 ? (kSlotsInEpi ? (kEpiFloats > kSlots ? kEpiFloats : kSlots) : 4 * TBN) : 4];
    __shared__ __attribute__((aligned(16))) float halo_own[MODE == 1 && !kSlotsInEpi ? TWAVES * kHalo * WN : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
    const int K = a.K;
    const int d = a.d;
    const int n_total = a.n_mats * d;
    const int n_tiles_n = (n_total + TBN - 1) / TBN;
    const int n_tiles_t = (int)((a.n_tok + TBT - 1) / TBT);
    int tile_n, tile_t;
    tile_of<MODE == 1 ? kGroupV : kGroupT>(blockIdx.x, gridDim.x, n_tiles_n, n_tiles_t, tile_n, tile_t);
    const int n0 = tile_n * TBN;
    // first token row of the tile
    // previous tile's last tokens (negative for the first tile: never stored)
    const int64_t t0 = (int64_t)tile_t * TBT;

    // ---- this lane's share of the block loads.  Wave w fills row blocks
    //      2w and 2w+1 of each operand.
    //      Lane l fills row l>>2 of the block, LDS chunk l&3, which holds
    //      global K chunk (l&3) ^ swz(row).  Token rows outside [0, n_tok) are
    //      clamped to a valid row: their products only reach outputs that the
    //      epilogue never writes, so no load leaves the buffers.
    const int lr = lane >> 2;
    const int lchunk = (lane & 3) ^ swz(lr);
    // d % 256 == 0, so a 256-row weight tile lies inside one matrix
    const int mat0 = min(n0, n_total - 1) / d;
    const char *wmat = reinterpret_cast<const char *>(pick(a.w, mat0));
    // operand row length (a split-K launch reads its share of longer rows)
    const int ld = (MODE == 3 && a.k_ld > 0) ? a.k_ld : K;
    const int kbase = kPlain ? (int)blockIdx.y * K : 0;
    // mode 4: operands [k_rows][w_ld] and [k_rows][e_ld]; k-rows past k_rows read as zeros
    const __amdgpu_buffer_rsrc_t wres =
        kKMajW ? make_rsrc(wmat, (uint32_t)(a.k_rows * a.w_ld * 2)) : make_rsrc(wmat, (uint32_t)d * ld * 2u);
    const __amdgpu_buffer_rsrc_t eres = kKMajE ? make_rsrc(a.emb, (uint32_t)(a.k_rows * a.e_ld * 2))
                                              : make_rsrc(a.emb, (uint32_t)(a.n_tok * ld * 2));
    // (a template-dependent bound here keeps the host pass from emitting the
    // kernel's launch stub, so the bound is the namespace constant both tiles share)
    static_assert(TBPW == kBlocksPerWave, "two row blocks per wave and operand in both tiles");
    // packed weights (forward modes): block blk of the tile is the matrix's
    // 16-row block (n0 - mat0 d) / 16 + blk, one 1 KB block per K stage; the
    // lane copies bytes 16 lane .. 16 lane + 15 of it (row lane / 4, already
    // swizzled), so the stage's weight offset is 1 KB per stage
    constexpr bool kFwdMode = MODE == 0 || MODE == 1 || MODE == 2;
    const bool wpk = kFwdMode && a.w_packed != 0;
    uint32_t woff[kBlocksPerWave], eoff[kBlocksPerWave];
#pragma unroll
    for (int i = 0; i < TBPW; ++i) {
        const int blk = wave * TBPW + i;
        const int row = blk * 16 + lr;
        // mode 1 takes the tokens of each group of four row blocks in the
        // order 4 * row + block (see the mode-1 epilogue)
        const int trow = MODE == 1 ? 64 * (blk >> 2) + 4 * lr + (blk & 3) : row;
        const int64_t t = min(max(t0 + trow, (int64_t)0), a.n_tok - 1);
        woff[i] = wpk ? (uint32_t)(((n0 - mat0 * d) / 16 + blk) * (K / 32) * 1024 + lane * 16)
                      : (uint32_t)((n0 - mat0 * d + row) * ld + lchunk * 8) * 2u;
        eoff[i] = (uint32_t)(t * ld + lchunk * 8) * 2u;
        if constexpr (kKMajW || kKMajE) {
            // instruction i of this wave fills k-rows RPI (TBPW wave + i) + lane / LPR,
            // LDS chunk lane % LPR of each, which holds the tile's column chunk
            // (lane % LPR) ^ 2 kswz(kr)
            constexpr int LPR = TBN / 8, RPI = 64 / LPR;
            const int kr = RPI * blk + lane / LPR;
            const int ch = (lane % LPR) ^ (2 * kswz<TBN / 16>(kr));
            if constexpr (kKMajW) woff[i] = (uint32_t)((int64_t)kr * a.w_ld + n0 + 8 * ch) * 2u;
            if constexpr (kKMajE) eoff[i] = (uint32_t)((int64_t)kr * a.e_ld + t0 + 8 * ch) * 2u;
        }
    }

    // Retrieval inside the launch (mode 2, TG): the slots of the tile's
    // tokens (tokens past n_tok: slot 0) and the table bases go to LDS
    // before the first stage.  A lane's 16-byte K
    // piece of stage s is element 32 s + 8 lchunk of E, i.e. element goff of
    // table gtau (d_e % 8 == 0: a piece never straddles two tables); the
    // stages are issued in K order, so (gtau, goff) advance by BK each.
    int gtau = 0, goff = 0;
    const int g_nt = kGather ? a.hc.n_tables : 0;
    const uint32_t g_row_bytes = kGather ? (uint32_t)(K / (g_nt > 0 ? g_nt : 1)) * 2u : 0u;
    if constexpr (kGather) {
        const int de = K / g_nt;
        const int32_t pad = a.hc.vocab_comp;
        const uint64_t Bv = (uint64_t)a.hc.vocab_comp + 1u;
        // one thread per token of the tile: its ids are read and compressed
        // once, then hashed into every table
        if (tid < TBT) {
            const int tl = tid;
            const int64_t tok = t0 + tl;
            const bool live_tok = tok < a.n_tok;
            int32_t c0 = pad, c1 = pad, c2 = pad;
            if (live_tok) {
                const int64_t b = tok / a.seqlen;
                const int32_t t = (int32_t)(tok - b * a.seqlen);
                const int32_t x0 = a.tokens[tok];
                c0 = compress_id(x0, a.comp_map, a.hc.vocab, pad);
                if (t >= 1) c1 = compress_id(a.tokens[tok - 1], a.comp_map, a.hc.vocab, pad);
                else c1 = a.prev_ctx ? a.prev_ctx[b * 2 + 1] : pad;
                if (t >= 2) c2 = compress_id(a.tokens[tok - 2], a.comp_map, a.hc.vocab, pad);
                else if (t == 1) c2 = a.prev_ctx ? a.prev_ctx[b * 2 + 1] : pad;
                else c2 = a.prev_ctx ? a.prev_ctx[b * 2 + 0] : pad;
                // one count per raw id: the blocks of the first weight tile
                if (a.bad && tile_n == 0 && (x0 < 0 || x0 >= a.hc.vocab)) atomicAdd(a.bad, 1u);
            }
            const uint64_t k2 = (uint64_t)c1 * Bv + (uint64_t)c0;
            const uint64_t k3 = ((uint64_t)c2 * Bv + (uint64_t)c1) * Bv + (uint64_t)c0;
            for (int tau = 0; tau < g_nt; ++tau) {
                const uint64_t key = a.hc.order_of[tau] == 2 ? k2 : k3;
                uint32_t *slots = kSlotsInEpi ? reinterpret_cast<uint32_t *>(taps_own) : idx_own;
                slots[tl * g_nt + tau] =
                    live_tok ? mod_prime(mix64(key ^ a.hc.seed[tau]), a.hc.rows[tau], a.hc.magic[tau]) : 0u;
            }
        }
        if (tid < g_nt) tab_s[tid] = pick(a.tables, tid);
        goff = 8 * lchunk;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool c = goff >= de;
            goff -= c ? de : 0;
            gtau += c ? 1 : 0;
        }
        __syncthreads();
    }

// The immediate offset of a buffer load with an LDS destination moves the LDS
// address as well, so the K position travels in the scalar offset, which only
// moves the global address.
#define ENGRAM_ISSUE(STG, k0)                                                                    \
    do {                                                                                         \
        const int kbytes = (kbase + (k0)) * 2;                                                   \
        const int kbw = wpk ? (k0) * 32 : kbytes; /* weight side: 1 KB per packed stage */      \
        if constexpr (kGather) {                                                                 \
            const char *tb = tab_s[gtau];                                                        \
            const uint32_t *slots = kSlotsInEpi ? reinterpret_cast<const uint32_t *>(taps_own) : idx_own; \
            _Pragma("unroll") for (int i = 0; i < TBPW; ++i) {                                   \
                const int blk = wave * TBPW + i;                                                 \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t *)&STG.w[blk * kBlockBytes], \
                                                         16, woff[i], kbw, 0, 0);                \
                const uint32_t ix = slots[(MODE == 1 ? 64 * (blk >> 2) + 4 * lr + (blk & 3)      \
                                                      : blk * 16 + lr) * g_nt + gtau];           \
                __builtin_amdgcn_global_load_lds(tb + (uint64_t)ix * g_row_bytes + 2 * goff,     \
                                                 (lds_void_t *)&STG.e[blk * kBlockBytes], 16, 0, 0); \
            }                                                                                    \
            goff += BK;                                                                          \
            _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                      \
                const bool c = goff >= (int)(g_row_bytes / 2u);                                  \
                goff -= c ? (int)(g_row_bytes / 2u) : 0;                                         \
                gtau += c ? 1 : 0;                                                               \
            }                                                                                    \
        } else if constexpr (kKMajW || kKMajE) {                                                 \
            /* mode 6: the weight side's k-rows are the stacked matrices' rows,                 \
               k_mat_rows per matrix, and a stage never straddles two */                          \
            __amdgpu_buffer_rsrc_t wr = wres;                                                    \
            int kw = (kbase + (k0)) * a.w_ld * 2;                                                \
            if constexpr (MODE == 6) {                                                           \
                const int kg = kbase + (k0), m6 = kg / a.k_mat_rows;                             \
                wr = make_rsrc(pick(a.w, m6), (uint32_t)a.k_mat_rows * a.w_ld * 2u);             \
                kw = (kg - m6 * a.k_mat_rows) * a.w_ld * 2;                                      \
            }                                                                                    \
            const int ke = kKMajE ? (kbase + (k0)) * a.e_ld * 2 : kbytes;                        \
            _Pragma("unroll") for (int i = 0; i < TBPW; ++i) {                                   \
                const int blk = wave * TBPW + i;                                                 \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_t *)&STG.w[blk * kBlockBytes], \
                                                         16, woff[i], kw, 0, 0);                 \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(eres, (lds_void_t *)&STG.e[blk * kBlockBytes], \
                                                         16, eoff[i], ke, 0, 0);                 \
            }                                                                                    \
        } else {                                                                                 \
            _Pragma("unroll") for (int i = 0; i < TBPW; ++i) {                                   \
                const int blk = wave * TBPW + i;                                                 \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t *)&STG.w[blk * kBlockBytes], \
                                                         16, woff[i], kbw, 0, 0);                \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(eres, (lds_void_t *)&STG.e[blk * kBlockBytes], \
                                                         16, eoff[i], kbytes, 0, 0);             \
            }                                                                                    \
        }                                                                                        \
    } while (0)
    constexpr int kLoadsPerStage = 2 * TBPW;  // per wave

    f32x4_t acc[FN][TFT];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < TFT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int wn_blk = (wave % TWGN) * (WN / 16);  // wave's first weight row block
    const int wt_blk = (wave / TWGN) * TFT;        // wave's first token row block
    const int fr = lane & 15;                    // fragment row
    const int fpos = fr * 64 + ((lane >> 4) ^ swz(fr)) * 16;  // byte offset inside a 1 KB block

    // mode 4 fragment of column block q: lane 16g + m takes k-rows 8g + 4h + m/4
    // (h = 0, 1), columns 16q + 4(m % 4) .. + 3 of each; the transposing read
    // hands lane 16g + m column 16q + m at k = 8g .. 8g + 7
    constexpr int kRowBytes = TBN * 2;
    int tr_row[2], tr_sw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kr = 8 * (lane >> 4) + 4 * h + ((lane & 15) >> 2);
        tr_row[h] = kr * kRowBytes + ((lane & 3) >> 1) * 16 + (lane & 1) * 8;
        tr_sw[h] = kswz<TBN / 16>(kr);
    }
    auto frag_tr = [&](const unsigned char *opnd, int q) -> bf16x8_t {
        const bf16x4_t lo = lds_read_tr(opnd + tr_row[0] + ((q ^ tr_sw[0]) << 5));
        const bf16x4_t hi = lds_read_tr(opnd + tr_row[1] + ((q ^ tr_sw[1]) << 5));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    (void)frag_tr;

#define ENGRAM_COMPUTE(STG)                                                                      \
    do {                                                                                         \
        bf16x8_t fa[FN], fb[TFT];                                                                 \
        if constexpr (kKMajW) {                                                                  \
            _Pragma("unroll") for (int i = 0; i < FN; ++i) fa[i] = frag_tr(STG.w, wn_blk + i);   \
        } else {                                                                                 \
            _Pragma("unroll") for (int i = 0; i < FN; ++i) fa[i] =                               \
                *reinterpret_cast<const bf16x8_t *>(&STG.w[(wn_blk + i) * kBlockBytes + fpos]);  \
        }                                                                                        \
        if constexpr (kKMajE) {                                                                  \
            _Pragma("unroll") for (int j = 0; j < TFT; ++j) fb[j] = frag_tr(STG.e, wt_blk + j);   \
        } else {                                                                                 \
            _Pragma("unroll") for (int j = 0; j < TFT; ++j) fb[j] =                               \
                *reinterpret_cast<const bf16x8_t *>(&STG.e[(wt_blk + j) * kBlockBytes + fpos]);  \
        }                                                                                        \
        _Pragma("unroll") for (int i = 0; i < FN; ++i)                                           \
            _Pragma("unroll") for (int j = 0; j < TFT; ++j)                                       \
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

    if constexpr (MODE == 1) {
        // gate of every row of the tile and branch (zero outside the tokens),
        // while the first stages are in flight
        for (int x = tid; x < BR * TBT; x += TTHREADS) {
            const int m = x / TBT, r = x - m * TBT;
            const int64_t t = t0 + r;
            alpha_s[m][r] = (t >= 0 && t < a.n_tok) ? a.alpha[m * a.n_tok + t] : 0.f;
        }
    }
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
    // Mode 0 epilogue input: h of the wave's TWT tokens x 128 channels, in
    // whole 128-byte rows (loading it straight into the MFMA layout would read
    // 16 rows x 32 bytes per instruction), two halves of TWT * 128 bytes for
    // channels nl + 64q.  Half 0 goes to buffers 0 and 1, half 1 to buffers 2
    // and 3 (wave w at byte w * kHalf of the pair); LDS row p is token tw + p,
    // its eight 16-byte pieces XOR-swizzled by hswz(p).  Half 0 is requested
    // as soon as buffers 0 and 1 are free, two stages before the main loop
    // ends.  Waves whose rows are not a W_k matrix send their requests past
    // the buffer's end (dropped, no branch), so every wave issues the same
    // number of loads.
    constexpr int kHalf = TWT * 128;
    constexpr int kStageBytes = 2 * TOPB;
    static_assert(TWAVES * kHalf <= 2 * kStageBytes, "half of every wave's h in two stage buffers");
    const int nw = n0 + wn_blk * 16;  // the wave's first output row (n_total % 128 == 0: inside the launch)
    const int mat = nw / d;           // the wave's 128 rows lie in one matrix (d % 128 == 0)
    const int nl = nw - mat * d;      // first channel within that matrix
    const int64_t tw = t0 + wt_blk * 16;
    auto hswz = [](int p) { return (p ^ (p >> 3)) & 7; };
    auto h_half = [&](int q) -> unsigned char * {
        const int off = wave * kHalf;
        unsigned char *pair0 = reinterpret_cast<unsigned char *>(q == 0 ? &st0 : &st2);
        unsigned char *pair1 = reinterpret_cast<unsigned char *>(q == 0 ? &st1 : &st3);
        return (off < kStageBytes ? pair0 : pair1) + (off % kStageBytes);
    };
    auto h_issue = [&](int q) {
        const bool is_k = mat < a.n_branches;
        const int hm = is_k ? mat : 0;
        const __amdgpu_buffer_rsrc_t hres = make_rsrc(
            reinterpret_cast<const uint16_t *>(a.h) + (int64_t)hm * a.n_tok * d, (uint32_t)(a.n_tok * d * 2));
        unsigned char *dst = h_half(q);
#pragma unroll
        for (int k = 0; k < TWT / 8; ++k) {
            const int p = 8 * k + (lane >> 3);
            const int64_t tok = min(tw + p, a.n_tok - 1);
            const uint32_t off = (uint32_t)((tok * d + nl) * 2) + (uint32_t)(((lane & 7) ^ hswz(p)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(hres, (lds_void_t *)(dst + k * 1024), 16,
                                                     is_k ? off : 0x80000000u, 128 * q, 0, 0);
        }
    };
    // Mode 1: chunk 0 of the epilogue (branch 0, the wave's first 64
    // channels) into buffer A, likewise two stages early.
    unsigned char *hA = reinterpret_cast<unsigned char *>(wave < 4 ? &st0 : &st1) + (wave & 3) * 8192;
    unsigned char *hB = reinterpret_cast<unsigned char *>(wave < 4 ? &st2 : &st3) + (wave & 3) * 8192;
    auto chunk0_issue = [&]() {
        const __amdgpu_buffer_rsrc_t hres = make_rsrc(a.h, (uint32_t)(a.n_tok * d * 2) * (uint32_t)BR);
        const int rowbase = 64 * (wave >> 1);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(hres, (lds_void_t *)(hA + k * 1024), 16,
                                                     chunk_offset(k, lane, rowbase, t0, a.n_tok, d, nl), 0, 0,
                                                     kCpolNT);
    };
    constexpr int kEarlyH = kGateK ? TWT / 8 : (MODE == 1 ? 8 : 0);  // loads issued in the ring's tail

    // the last four stages: ks = k_steps - 4; stages ks..ks+2 are in flight
    wait_vmcnt<2 * kLoadsPerStage>();
    block_barrier();
    ENGRAM_ISSUE(st3, (ks + 3) * BK);
    ENGRAM_COMPUTE(st0);
    wait_vmcnt<2 * kLoadsPerStage>();
    block_barrier();
    ENGRAM_COMPUTE(st1);
    wait_vmcnt<kLoadsPerStage>();
    block_barrier();  // buffers 0 and 1 are done with
    if constexpr (kGateK) h_issue(0);
    if constexpr (MODE == 1) chunk0_issue();
    ENGRAM_COMPUTE(st2);
    wait_vmcnt<kEarlyH>();
    block_barrier();
    ENGRAM_COMPUTE(st3);
#undef ENGRAM_COMPUTE
#undef ENGRAM_ISSUE

    // ---- epilogue.  acc[i][j][r] is output channel n = nw + 16i + 4*(lane/16) + r
    //      of token t = tw + 16j + lane%16.
    const int sub = 4 * (lane >> 4);

    // gate partials first (mode 5 then also stores k): the partial sums wait
    // for all of this wave's memory operations, which the stores would join
    if constexpr (kGateK) {
    if (mat < a.n_branches) {
        // gate partials of branch `mat` over channels [nl, nl+128).
        // gamma_h * gamma_k for the wave's channels goes through LDS, so it
        // costs no registers; each wave writes and reads only its own 512 bytes.
        float *gsm = gsm_s + wave * WN;
        {
            const float *gh = pick(a.gamma_h, mat);
            const float *gk = pick(a.gamma_k, mat);
            for (int c = lane; c < WN; c += 64) gsm[c] = gh[nl + c] * gk[nl + c];
        }
        const int part = nl / kPartCols;
        float *pbase = a.partials + ((int64_t)mat * a.n_parts + part) * 3 * a.n_tok;
        // half 1 of h (half 0 is in flight since the ring's tail)
        block_barrier();  // every wave is done reading the stage buffers
        h_issue(1);
        unsigned char *h0 = h_half(0), *h1 = h_half(1);
        // Half 0's channels (i < FN/2) are summed while half 1 is in flight,
        // then half 1's: each token's sums still add i = 0..FN-1 in order.
        float s_hk[TFT], s_kk[TFT], s_hh[TFT];
        auto add_half = [&](auto hc) {
            constexpr int H = decltype(hc)::value;
#pragma unroll
            for (int j = 0; j < TFT; ++j) {
                const int p = 16 * j + (lane & 15);
                if (H == 0) s_hk[j] = s_kk[j] = s_hh[j] = 0.f;
#pragma unroll
                for (int i = H * (FN / 2); i < (H + 1) * (FN / 2); ++i) {
                    const u32x2_t x = *reinterpret_cast<const u32x2_t *>(
                        (H ? h1 : h0) + p * 128 + (((2 * (i & 3) + (sub >> 3)) ^ hswz(p)) << 4) + (sub & 4) * 2);
                    const f32x4_t g = *reinterpret_cast<const f32x4_t *>(gsm + 16 * i + sub);
                    const float h4[4] = {bf16_to_f32(x[0] & 0xFFFFu), bf16_to_f32(x[0] >> 16),
                                         bf16_to_f32(x[1] & 0xFFFFu), bf16_to_f32(x[1] >> 16)};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float kv = acc[i][j][r];
                        s_hk[j] += h4[r] * g[r] * kv;
                        s_kk[j] += kv * kv;
                        s_hh[j] += h4[r] * h4[r];
                    }
                }
            }
        };
        static_assert(FN == 8, "two halves of four 16-channel blocks");
        wait_vmcnt<TWT / 8>();  // half 0 (half 1's TWT/8 loads may be in flight)
        asm volatile("" ::: "memory");
        add_half(std::integral_constant<int, 0>{});
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        add_half(std::integral_constant<int, 1>{});
#pragma unroll
        for (int j = 0; j < TFT; ++j) {
            const int64_t t = tw + 16 * j + (lane & 15);
            float s_hk_j = s_hk[j], s_kk_j = s_kk[j], s_hh_j = s_hh[j];
            // the four lanes {l, l+16, l+32, l+48} hold the same token
            s_hk_j += __shfl_xor(s_hk_j, 16); s_hk_j += __shfl_xor(s_hk_j, 32);
            s_kk_j += __shfl_xor(s_kk_j, 16); s_kk_j += __shfl_xor(s_kk_j, 32);
            s_hh_j += __shfl_xor(s_hh_j, 16); s_hh_j += __shfl_xor(s_hh_j, 32);
            if (lane < 16 && t < a.n_tok) {
                pbase[t] = s_hk_j;
                pbase[a.n_tok + t] = s_kk_j;
                pbase[2 * a.n_tok + t] = s_hh_j;
            }
        }
    } else if constexpr (!kPlain) {
        // v = W_v e, kept fp32 [n_tok][d]: rounding it to bf16 here would add
        // up to half a bf16 ulp of |v| to every gated value the conv sums.
#pragma unroll
        for (int j = 0; j < TFT; ++j) {
            const int64_t t = tw + 16 * j + (lane & 15);
            if (t >= a.n_tok) continue;
#pragma unroll
            for (int i = 0; i < FN; ++i)
                *reinterpret_cast<f32x4_t *>(a.v + t * d + nl + 16 * i + sub) = acc[i][j];
        }
    }
    }
    if constexpr (kPlain) {
        // plain contraction: every tile stores its fp32 block, four
        // consecutive rows n (16 bytes) of one token t per lane and block
        float *out = a.out_f32 + (int64_t)blockIdx.y * a.out_split;
#pragma unroll
        for (int j = 0; j < TFT; ++j) {
            const int64_t t = tw + 16 * j + (lane & 15);
            if (t >= a.n_tok) continue;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int n = nw + 16 * i + sub;
                if (n < a.n_rows) *reinterpret_cast<f32x4_t *>(out + t * a.out_ld + n) = acc[i][j];
            }
        }
    } else if constexpr (!kGateK) {
        // each wave's two chunk buffers: 8 KB of st0/st1 (A) and of st2/st3 (B)
        if constexpr (kSlotsInEpi)
            fused_value_epilogue<BR, SILU>(a, acc, alpha_s, taps_own + 4 * TBN, taps_own, hA, hB, wave, lane, nl, n0,
                                           tile_t, t0);
        else
            fused_value_epilogue<BR, SILU>(a, acc, alpha_s, halo_own, taps_own, hA, hB, wave, lane, nl, n0, tile_t,
                                           t0);
    }
}

// [rows][K] bf16 -> packed operand blocks: thread p writes 16-byte piece p,
// piece c % 4 of row (c / 4) % 16 of block c / 64 = (row block, K stage),
// which holds the row's values 8 q .. 8 q + 7 of that stage for
// q = (c % 4) ^ swz(row).
__global__ __launch_bounds__(256) void pack_weight_kernel(const u32x4_t *__restrict__ w, u32x4_t *__restrict__ out,
                                                          int64_t pieces, int32_t K) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= pieces) return;
    const int stages = K / 32;
    const int64_t blk = c >> 6;
    const int r = (int)((c >> 2) & 15), pos = (int)(c & 3);
    const int64_t rb = blk / stages;
    const int st = (int)(blk - rb * stages);
    const int q = pos ^ swz(r);
    out[c] = w[((rb * 16 + r) * K + 32 * st + 8 * q) / 8];
}

}  // namespace

void launch_pack_weight(const void *w, void *packed, int32_t rows, int32_t K, hipStream_t s) {
    const int64_t pieces = (int64_t)rows * K / 8;
    launch_kernel(pack_weight_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), s,
                  static_cast<const u32x4_t *>(w), static_cast<u32x4_t *>(packed), pieces, K);
}

void launch_proj_bf16(const ProjArgs &a, hipStream_t s) {
    const int n_total = a.n_mats * a.d;
    const int64_t wide = (int64_t)((n_total + BN - 1) / BN) * ((a.n_tok + BT - 1) / BT);
    if (wide < 256) {  // fewer wide tiles than CUs: narrow tiles, up to two per CU
        const int64_t blocks = (int64_t)((n_total + 127) / 128) * ((a.n_tok + 127) / 128);
        launch_kernel((proj_bf16_kernel<0, 1, false, true>), dim3((unsigned)blocks), dim3(256), s, a);
    } else {
        launch_kernel((proj_bf16_kernel<0, 1, false, false>), dim3((unsigned)wide), dim3(kThreads), s, a);
    }
}

// 256 x 256 tiles when they (times the K splits) occupy at least three
// quarters of the CUs in a round; else 128 x 128 tiles, two per CU
static bool plain_wide(int64_t wide_blocks, int splits) { return wide_blocks * splits >= 192; }

void launch_proj_plain_bf16(const ProjArgs &a, hipStream_t s, int splits) {
    const int n_total = a.n_mats * a.d;
    const int64_t wide = (int64_t)((n_total + BN - 1) / BN) * ((a.n_tok + BT - 1) / BT);
    if (!plain_wide(wide, splits)) {
        const int64_t blocks = (int64_t)((n_total + 127) / 128) * ((a.n_tok + 127) / 128);
        launch_kernel((proj_bf16_kernel<3, 1, false, true>), dim3((unsigned)blocks, (unsigned)splits), dim3(256), s,
                      a);
    } else {
        launch_kernel((proj_bf16_kernel<3, 1, false, false>), dim3((unsigned)wide, (unsigned)splits),
                      dim3(kThreads), s, a);
    }
}

void launch_proj_kv_partials_bf16(const ProjArgs &a, hipStream_t s) {
    const int n_total = a.n_mats * a.d;
    const int64_t wide = (int64_t)((n_total + BN - 1) / BN) * ((a.n_tok + BT - 1) / BT);
    if (wide < 256) {
        const int64_t blocks = (int64_t)((n_total + 127) / 128) * ((a.n_tok + 127) / 128);
        launch_kernel((proj_bf16_kernel<5, 1, false, true>), dim3((unsigned)blocks), dim3(256), s, a);
    } else {
        launch_kernel((proj_bf16_kernel<5, 1, false, false>), dim3((unsigned)wide), dim3(kThreads), s, a);
    }
}

void launch_proj_plain_kmajor_w_bf16(const ProjArgs &a, hipStream_t s) {
    const int n_total = a.n_mats * a.d;
    const int64_t wide = (int64_t)((n_total + BN - 1) / BN) * ((a.n_tok + BT - 1) / BT);
    if (!plain_wide(wide, 1)) {
        const int64_t blocks = (int64_t)((n_total + 127) / 128) * ((a.n_tok + 127) / 128);
        launch_kernel((proj_bf16_kernel<6, 1, false, true>), dim3((unsigned)blocks), dim3(256), s, a);
    } else {
        launch_kernel((proj_bf16_kernel<6, 1, false, false>), dim3((unsigned)wide), dim3(kThreads), s, a);
    }
}

void launch_proj_plain_kmajor_bf16(const ProjArgs &a, hipStream_t s, int splits) {
    const int n_total = a.n_mats * a.d;
    const int64_t wide = (int64_t)((n_total + BN - 1) / BN) * ((a.n_tok + BT - 1) / BT);
    if (!plain_wide(wide, splits)) {
        const int64_t blocks = (int64_t)((n_total + 127) / 128) * ((a.n_tok + 127) / 128);
        launch_kernel((proj_bf16_kernel<4, 1, false, true>), dim3((unsigned)blocks, (unsigned)splits), dim3(256), s,
                      a);
    } else {
        launch_kernel((proj_bf16_kernel<4, 1, false, false>), dim3((unsigned)wide, (unsigned)splits),
                      dim3(kThreads), s, a);
    }
}

bool proj_gather_ok(const ProjArgs &a, int32_t n_tables) {
    const int n_total = a.n_mats * a.d;
    const int64_t wide = (int64_t)((n_total + BN - 1) / BN) * ((a.n_tok + BT - 1) / BT);
    return wide < 256 && n_tables >= 1 && n_tables <= kGatherMaxTables && a.K % n_tables == 0 &&
           (a.K / n_tables) % 8 == 0;
}

void launch_proj_gather_bf16(const ProjArgs &a, hipStream_t s) {
    const int n_total = a.n_mats * a.d;
    const int64_t blocks = (int64_t)((n_total + 127) / 128) * ((a.n_tok + 127) / 128);
    launch_kernel((proj_bf16_kernel<2, 1, false, true>), dim3((unsigned)blocks), dim3(256), s, a);
}

int plain_k_splits(int64_t n_tok, int64_t rows, int64_t K) {
    auto can_double = [&](int splits) { return K % (128 * splits * 2) == 0 && K / (splits * 2) >= 1024; };
    // wide tiles, one workgroup per CU: split until a round is (nearly) full
    const int64_t wide = ((rows + 255) / 256) * ((n_tok + 255) / 256);
    int splits = 1;
    while (wide * splits * 2 <= 256 && can_double(splits)) splits *= 2;
    if (plain_wide(wide, splits)) return splits;
    // narrow tiles run two workgroups per CU: 512 fill the chip once
    const int64_t narrow = ((rows + 127) / 128) * ((n_tok + 127) / 128);
    splits = 1;
    while (narrow * splits * 2 <= 512 && can_double(splits)) splits *= 2;
    return splits;
}

namespace {

template <bool TG>
void launch_proj_v_fused(const ProjArgs &a, hipStream_t s) {
    const int n_tiles_n = (a.d + BN - 1) / BN;
    const int64_t n_tiles_t = (a.n_tok + BT - 1) / BT;
    const dim3 grid((unsigned)((int64_t)n_tiles_n * n_tiles_t));
#define ENGRAM_PROJ_V_LAUNCH(BR)                                                                      \
    do {                                                                                              \
        if (a.conv_mode == ENGRAM_CONV_SILU_SKIP)                                                     \
            launch_kernel((proj_bf16_kernel<1, BR, true, false, TG>), grid, dim3(kThreads), s, a);    \
        else                                                                                          \
            launch_kernel((proj_bf16_kernel<1, BR, false, false, TG>), grid, dim3(kThreads), s, a);   \
    } while (0)
    switch (a.n_branches) {
        case 1: ENGRAM_PROJ_V_LAUNCH(1); break;
        case 2: ENGRAM_PROJ_V_LAUNCH(2); break;
        case 3: ENGRAM_PROJ_V_LAUNCH(3); break;
        default: ENGRAM_PROJ_V_LAUNCH(4); break;
    }
#undef ENGRAM_PROJ_V_LAUNCH
}

}  // namespace

void launch_proj_v_fused_bf16(const ProjArgs &a, hipStream_t s) { launch_proj_v_fused<false>(a, s); }

bool proj_gather_tables_ok(const ProjArgs &a, int32_t n_tables) {
    return n_tables >= 1 && n_tables <= kGatherMaxTables && a.K % n_tables == 0 && (a.K / n_tables) % 8 == 0;
}

void launch_proj_k_gather_bf16(const ProjArgs &a, hipStream_t s) {
    const int n_total = a.n_mats * a.d;
    const int64_t wide = (int64_t)((n_total + BN - 1) / BN) * ((a.n_tok + BT - 1) / BT);
    if (wide < 256) {  // the tiles launch_proj_bf16 would take: 128 x 128
        launch_proj_gather_bf16(a, s);
        return;
    }
    launch_kernel((proj_bf16_kernel<0, 1, false, false, true>), dim3((unsigned)wide), dim3(kThreads), s, a);
}

void launch_proj_v_fused_gather_bf16(const ProjArgs &a, hipStream_t s) { launch_proj_v_fused<true>(a, s); }

}  // namespace engram
