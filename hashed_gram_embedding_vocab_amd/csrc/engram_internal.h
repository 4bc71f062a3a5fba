// engram_internal.h -- shared declarations of the gfx950 kernels and their
// host-side launchers.  Not part of the public ABI (see include/engram.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"
#include "hash_math.h"

namespace engram {

// ---------------------------------------------------------------- launches
// Events of the launch being timed (profiling on), else null.  Every kernel
// of the library is launched through launch_kernel, which hands them to
// hipExtLaunchKernel: the dispatch packet itself takes the timestamps, so
// timing adds no packets to the stream.  The start event goes to the first
// kernel of a timed launch, the stop event to every kernel (the last wins).
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents &launch_events();  // this thread's

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
    LaunchEvents &ev = launch_events();
    hipEvent_t start = ev.start;
    ev.start = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, ev.stop, 0, args...);
}

constexpr int kMaxTables = ENGRAM_MAX_TABLES;
constexpr int kMaxBranches = ENGRAM_MAX_BRANCHES;

// Clang vector types (HIP's uint4/float4 are unions that defeat scalar
// replacement when kept in arrays, which then land in scratch or LDS).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 bits
// bf16 values travel as raw 16-bit patterns; widening is a shift, narrowing
// rounds to nearest even (finite values only: every value on the path is).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// ---------------------------------------------------------------- hashing
// mix64, table_seed, mod_magic and mod_prime: hash_math.h

// Vocabulary projection of one raw id; ids outside [0, vocab) become PAD.
__device__ __forceinline__ int32_t compress_id(int32_t x, const int32_t *__restrict__ comp_map,
                                               int32_t vocab, int32_t pad) {
    return (x >= 0 && x < vocab) ? __ldg(comp_map + x) : pad;
}

struct HashConsts {
    uint64_t seed[kMaxTables];   // per-table 64-bit seed s_tau
    uint64_t magic[kMaxTables];  // floor((2^64-1) / rows_tau), for the Barrett reduction
    uint32_t rows[kMaxTables];   // prime row counts
    int32_t order_of[kMaxTables];// n-gram order of table tau (2 or 3)
    int32_t n_tables;
    int32_t vocab;
    int32_t vocab_comp;
};

void launch_hash(const HashConsts &hc, const int32_t *tokens, int32_t batch, int32_t seqlen,
                 const int32_t *comp_map, const int32_t *prev_ctx, uint32_t *idx,
                 uint32_t *bad, hipStream_t s);


// ---------------------------------------------------------------- gather
struct GatherConsts {
    const char *table[kMaxTables];
    uint32_t last_row[kMaxTables];
    int32_t n_tables;
    int32_t row_chunks;   // 16-byte chunks per table row
    int32_t tok_chunks;   // 16-byte chunks per token (n_tables * row_chunks)
    uint64_t magic_tok;   // division by tok_chunks (0 when tok_chunks == 1)
    uint64_t magic_row;   // division by row_chunks (0 when row_chunks == 1)
};

void launch_gather(const GatherConsts &gc, const uint32_t *idx, int64_t n_tok, void *emb,
                   hipStream_t s);
// Tables in host memory with a hot-row cache in HBM: the cache of table tau
// is capacity slots of keys (row + 1, 0 = free; open addressing, linear
// probing) and rows [capacity][d_e].  capacity 0: no cache.
void launch_cache_build(const GatherConsts &gc, uint32_t capacity, const uint32_t *hot, int32_t n_hot,
                        uint32_t *keys, void *rows, hipStream_t s);
// max_workgroups > 0 caps the launch; each workgroup then loops over its
// share of the token groups
void launch_cached_gather(const GatherConsts &gc, uint32_t capacity, const uint32_t *idx, int64_t n_tok,
                          const uint32_t *keys, const void *rows, void *emb, int32_t max_workgroups,
                          hipStream_t s);
// Host-gather prefetch: E assembled from cache rows and staged miss rows
// (code[pair] = cache slot, or 0x80000000 | staged row).
void launch_prefetch_assemble(const GatherConsts &gc, int64_t n_tok, const uint32_t *code, const void *cache_rows,
                              const void *staged, void *emb, hipStream_t s);
// Retrieval in one pass (engram_forward): every lane hashes the n-gram of its
// own (token, table) pair and copies its 16-byte chunk of that row.
// ctx_out: roll this carried context (the prev_ctx array) inside the launch;
// honoured only when seqlen == 1, else ignored
void launch_hash_gather(const HashConsts &hc, const GatherConsts &gc, const int32_t *tokens,
                        int32_t batch, int32_t seqlen, const int32_t *comp_map,
                        const int32_t *prev_ctx, uint32_t *bad, void *emb, hipStream_t s,
                        int32_t *ctx_out = nullptr);

// ---------------------------------------------------------------- projections
struct ProjArgs {
    const void *emb;                       // [n_tok][K]
    const void *w[kMaxBranches + 1];       // the launch's weight matrices stacked along N, each [d][K]
    const void *h;                         // [B_r][n_tok][d]
    const float *gamma_h[kMaxBranches];
    const float *gamma_k[kMaxBranches];
    float *partials;                       // [B_r][n_parts][3][n_tok]
    float *v;                              // [n_tok][d] fp32
    float *kbuf;                           // f32 path only: [B_r][n_tok][d]
    int64_t n_tok;
    int32_t K;                             // D_e
    int32_t d;
    int32_t n_branches;
    int32_t n_parts;
    int32_t n_mats;                        // matrices in w[]: mat < n_branches is W_k^(mat), else W_v
    // fused value launch only (gate, gated value, conv, residual in the epilogue)
    void *out;                             // [B_r][n_tok][d]
    const float *conv_w;                   // [d][K_c]
    const void *conv_state;                // [B_r][batch][K_c-1][d] fp32 (bf16 if state_bf16) or null
    float *state_stage;                    // [B_r][batch][K_c-1][d] fp32 or null
    int32_t state_bf16;                    // conv_state holds bf16 values
    const float *alpha;                    // [B_r][n_tok], from the gate kernel
    float *seam_v;                         // [token tiles][6][d] fp32 v of each tile's first and last 3 rows
    int32_t batch, seqlen, conv_k, conv_mode;
    uint32_t flags;
    // plain launch only (mode 3): C[t][n] = sum_k W[n][k] E[t][k] stored fp32
    float *out_f32;                        // element (t, n) at out_f32[t * out_ld + n]
    int64_t out_ld;
    int32_t n_rows;                        // rows of W to store (n < n_rows)
    // split K: launch z contracts k in [z K, (z+1) K) of rows k_ld long and
    // stores at out_f32 + z * out_split (k_ld 0: one launch, rows K long)
    int32_t k_ld;
    int64_t out_split;
    // mode 4 (both operands K-major): w[0] is [k_rows][w_ld] and emb
    // [k_rows][e_ld]; row k of each holds that k for every column
    int64_t k_rows;
    int32_t w_ld, e_ld;
    // mode 6 (weight side K-major): k-row n of the stacked w[] is row
    // n % k_mat_rows of matrix n / k_mat_rows, each [k_mat_rows][w_ld]
    int32_t k_mat_rows;
    // retrieval inside the launch (mode 2): every block hashes its tokens'
    // n-grams and reads its E operand straight from the table rows
    const int32_t *tokens;                 // [batch][seqlen] raw ids
    const int32_t *comp_map;               // [V]
    const int32_t *prev_ctx;               // [batch][2] or null
    uint32_t *bad;                         // counter of raw ids outside [0, V), or null
    const char *tables[kMaxTables];
    HashConsts hc;
    // forward modes (0-2): every w[] matrix is in the packed operand layout
    // (engram_pack_weight), each ring stage's weight blocks one 1 KB read
    int32_t w_packed;
};

// [rows][K] bf16 -> the packed operand layout of engram_pack_weight
// (rows % 16 == 0, K % 32 == 0)
void launch_pack_weight(const void *w, void *packed, int32_t rows, int32_t K, hipStream_t s);

constexpr int kPartCols = 128;  // columns of d summed into one gate partial (bf16 path)

// W_k^(m) (and, when n_mats == n_branches + 1, W_v) projections: gate
// partials from W_k tiles, fp32 v from W_v tiles.
void launch_proj_bf16(const ProjArgs &a, hipStream_t s);
// The same launch (W_k of every branch and W_v, gate partials and fp32 v)
// with retrieval inside: each block hashes the n-grams of its tokens and
// loads E straight from the tables into its operand ring, so E never reaches
// memory.  Only where launch_proj_bf16 takes 128 x 128 tiles and
// n_tables <= kGatherMaxTables (proj_gather_ok).
constexpr int kGatherMaxTables = 16;
bool proj_gather_ok(const ProjArgs &a, int32_t n_tables);
void launch_proj_gather_bf16(const ProjArgs &a, hipStream_t s);
// W_v projection with the gate, gated value, depthwise causal conv, residual
// and conv-state update fused into the epilogue (needs seqlen >= K_c - 1).
// Rows 0..2 of each 256-token tile whose conv history lies in the previous
// tile are left to launch_seam.
constexpr int kTokTile = 256;
void launch_proj_v_fused_bf16(const ProjArgs &a, hipStream_t s);
// Retrieval inside the two launches of the route above (W_v separate): the
// W_k launch of every branch and the fused W_v launch each hash the n-grams
// of their tiles' tokens and read their E operand from the tables, as
// launch_proj_gather_bf16 does (E never reaches memory; the W_k launch takes
// 128 x 128 tiles where launch_proj_bf16 would).  Only the launch given
// a.bad counts out-of-range ids; neither writes the carried context.  Needs
// n_tables <= kGatherMaxTables and d_e % 8 == 0 (proj_gather_tables_ok).
bool proj_gather_tables_ok(const ProjArgs &a, int32_t n_tables);
void launch_proj_k_gather_bf16(const ProjArgs &a, hipStream_t s);
void launch_proj_v_fused_gather_bf16(const ProjArgs &a, hipStream_t s);
// Plain contraction C[t][n] = sum_k W[n][k] E[t][k] (bf16 operands, fp32
// accumulate and result) on the same MFMA main loop: W rows are the n_mats
// matrices of a.w stacked (a.d rows each), E has a.n_tok rows, K = a.K
// (K % 128 == 0); rows n >= a.n_rows and tokens t >= a.n_tok are not stored.
// splits > 1: a.K is the share of each of the splits launches (a.k_ld =
// splits * a.K), each storing its own partial result (see ProjArgs).
void launch_proj_plain_bf16(const ProjArgs &a, hipStream_t s, int splits = 1);
// The same contraction with both operands stored K-major: C[t][n] = sum_k
// w[0][k][n] emb[k][t] over k in [z K, (z+1) K) for launch z of `splits`
// (k-rows past k_rows count as zero); fp32 out as above.  K % 128 == 0,
// w_ld, e_ld and the column counts multiples of 8.
void launch_proj_plain_kmajor_bf16(const ProjArgs &a, hipStream_t s, int splits = 1);
// C[t][n] = sum_k W[k][n] emb[t][k] with the k-rows of W taken from the
// stacked matrices w[0..] (k_mat_rows rows of w_ld each; k_mat_rows % 32 == 0),
// emb K-contiguous as in mode 3; fp32 out, no split.
void launch_proj_plain_kmajor_w_bf16(const ProjArgs &a, hipStream_t s);
// The plain contraction over the stacked [W_k^(m); W_v] (n_mats = n_branches
// + 1, K = D_e, no split) that also leaves, for the W_k rows, the gate
// partial sums of launch_proj_bf16 (h, gamma_h, gamma_k, partials, n_parts).
void launch_proj_kv_partials_bf16(const ProjArgs &a, hipStream_t s);
// How many K splits fill the chip for a plain contraction of n_tok x rows
// outputs over K (a power of two; K / splits stays a multiple of 128).
int plain_k_splits(int64_t n_tok, int64_t rows, int64_t K);
void launch_proj_f32(const ProjArgs &a, hipStream_t s);  // k into kbuf, v, then partials

// ---------------------------------------------------------------- fusion
// The carried context of the next chunk: the last two compressed ids of
// (prev_ctx followed by this chunk's tokens), per sequence.  engram_forward
// hands it to a kernel that runs after retrieval has read prev_ctx.
struct CtxUpdate {
    const int32_t *tokens;     // [batch][seqlen] raw ids
    const int32_t *comp_map;   // [vocab]
    int32_t *prev_ctx;         // [batch][2], or null: nothing to update
    int32_t vocab, vocab_comp;
};

__device__ __forceinline__ void ctx_update_one(const CtxUpdate &c, int32_t b, int32_t seqlen) {
    const int32_t *seq = c.tokens + (int64_t)b * seqlen;
    const int32_t n1 = compress_id(seq[seqlen - 1], c.comp_map, c.vocab, c.vocab_comp);
    const int32_t n0 =
        seqlen >= 2 ? compress_id(seq[seqlen - 2], c.comp_map, c.vocab, c.vocab_comp) : c.prev_ctx[b * 2 + 1];
    c.prev_ctx[b * 2 + 0] = n0;
    c.prev_ctx[b * 2 + 1] = n1;
}

void launch_ctx_update(const CtxUpdate &c, int32_t batch, int32_t seqlen, hipStream_t s);

// Gate per branch and token, alpha = sigmoid(<RMSNorm(h), RMSNorm(k)> / sqrt(d)),
// from the partial sums of the W_k projection (summed in a fixed order).
struct GateArgs {
    const float *partials;     // [B_r][n_parts][3][n_tok]
    float *alpha;              // [B_r][n_tok]
    int64_t n_tok;
    int32_t d, n_branches, n_parts;
    float eps;
    CtxUpdate ctx;             // done by the first batch threads of branch 0
    int32_t batch, seqlen;
};

void launch_gate(const GateArgs &a, hipStream_t s);

// The rows launch_proj_v_fused_bf16 leaves: tile rows 0..2 (tile > 0) whose
// conv history reaches into the previous tile, from both tiles' saved v.
struct SeamArgs {
    const float *seam_v;       // [n_tiles][6][d]
    const float *alpha;        // [B_r][n_tok]
    const void *h;             // [B_r][n_tok][d] bf16
    void *out;                 // [B_r][n_tok][d] bf16
    const float *conv_w;       // [d][K_c]
    const void *conv_state;    // [B_r][batch][K_c-1][d] fp32 (bf16 if state_bf16) or null
    int64_t n_tok;
    int32_t n_tiles, batch, seqlen, d, n_branches, conv_k, conv_mode;
    uint32_t flags;
    int32_t state_bf16;
};

void launch_seam(const SeamArgs &a, hipStream_t s);

constexpr int kFusePositions = 32;  // positions of one sequence per fusion-kernel workgroup

struct FuseArgs {
    const float *v;            // [n_tok][d] fp32
    const float *partials;     // [B_r][n_parts][3][n_tok]: the gate is computed here
    float *alpha;              // [B_r][n_tok] gate output, or null
    const void *h;             // [B_r][n_tok][d]
    void *out;                 // [B_r][n_tok][d]
    const float *conv_w;       // [d][K_c]
    const void *conv_state;    // [B_r][batch][K_c-1][d] fp32 (bf16 if state_bf16) or null
    void *state_stage;         // [B_r][batch][K_c-1][d] fp32 (bf16 if stage_bf16) or null
    int32_t state_bf16;        // conv_state holds bf16 values
    int32_t stage_bf16;        // state_stage is the bf16 conv state itself (updated in place)
    int32_t batch, seqlen, d, n_branches, n_parts, conv_k, conv_mode;
    float eps;
    uint32_t flags;
    CtxUpdate ctx;             // done by the first workgroup of each sequence
};

void launch_fuse(const FuseArgs &a, engram_dtype dt, hipStream_t s);

// ---------------------------------------------------------------- backward
struct BwdArgs {
    const void *h;                          // [B_r][n_tok][d] bf16
    const void *dout;                       // [B_r][n_tok][d] bf16
    void *dh;                               // [B_r][n_tok][d] bf16 (out)
    const float *kv;                        // [n_tok][kv_ld]: k of every branch, then v (fp32)
    int64_t kv_ld;                          // (B_r + 1) d
    float *stats;                           // [4][B_r][n_tok]: rh, rk, s, alpha
    const float *partials;                  // [B_r][n_parts][3][n_tok]: the k/v projection's gate partials
    int32_t n_parts;                        // d / 128
    float *dalpha_part;                     // [B_r][n_stripes][n_tok]
    float *dconv_part;                      // [conv blocks][d][K_c]
    float *dg_part;                         // [2][B_r][gate chunks][d]: gamma_h, then gamma_k
    uint16_t *dkv;                          // [n_tok][dkv_ld] bf16: dk of every branch, then dv
    int64_t dkv_ld;                         // (B_r + 1) d
    const float *gamma_h[kMaxBranches];
    const float *gamma_k[kMaxBranches];
    const float *conv_w;                    // [d][K_c]
    int64_t n_tok;
    int32_t batch, seqlen, d, n_branches, conv_k, conv_mode;
    int32_t n_stripes;                      // ceil(d / 1024)
    uint32_t flags;
    float eps;
};
void launch_bwd_gate_stats(const BwdArgs &a, hipStream_t s);
void launch_bwd_conv(const BwdArgs &a, hipStream_t s);
void launch_bwd_gate(const BwdArgs &a, hipStream_t s);
int32_t bwd_conv_blocks(int32_t batch, int32_t seqlen);
int32_t bwd_gate_chunks(int64_t n_tok);
// out[g][i] = sum over r of in[g][r][i] in a fixed order (rows split into
// bwd_sum_slabs(rows) slabs, each summed into part[g][slab][i] first)
int32_t bwd_sum_slabs(int64_t rows);
void launch_bwd_sum_rows(const float *in, int64_t groups, int64_t rows, int64_t width, float *part, float *out,
                         hipStream_t s);
// out[g][i] = sum over s = 0..S-1, ascending, of part[g][s][i]
void launch_bwd_sum_parts(const float *part, int64_t groups, int64_t width, int32_t S, float *out, hipStream_t s);

struct BwdTableArgs {
    const uint32_t *idx;                    // [n_tok][n_tables]
    const float *demb;                      // [n_tok][n_tables * head_dim]
    int64_t n_tok;
    int32_t n_tables, head_dim;
    const uint32_t *table_rows;             // [n_tables] rows of each table
    void *keys_in, *keys_out;               // [n_tables * n_tok], 32- or 64-bit keys (8 bytes each reserved)
    uint32_t *vals_in, *vals_out, *head, *incl;
    void *temp;                             // sort / scan scratch
    size_t temp_bytes;
    uint32_t *row_ids;
    float *row_grads;
    int32_t *row_counts;
    // per 64-item chunk of the sorted items: partial sums of the runs that
    // cross its start (lead) and its end (tail), flags, tail slot and row
    float *lead, *tail;                     // [chunks][head_dim]
    uint32_t *cflags;                       // [chunks]
    uint32_t *tinfo;                        // [chunks][2]
};
int64_t bwd_row_chunks(int64_t n_items);
size_t bwd_table_temp_bytes(int64_t n_items);
hipError_t launch_bwd_table_grad(const BwdTableArgs &t, hipStream_t s);

// ---------------------------------------------------------------- synthetic tables
// ---------------------------------------------------------------- copies
void launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t s);  // n % 4 == 0
// dst[i] = src[i] rounded to nearest-even bf16 (n % 4 == 0)
void launch_f32_to_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t s);

void launch_synth_fill(engram_dtype dt, uint64_t seed, int32_t tau, int64_t rows, int32_t head_dim,
                       void *table, hipStream_t s);
// Streaming read (mode 0) or copy (mode 1) of bytes (a multiple of 16);
// false if unroll is not 4, 8 or 16.
bool launch_stream_probe(int mode, bool nontemporal, int unroll, const void *src, void *dst, int64_t bytes,
                         int blocks, hipStream_t s);

}  // namespace engram
