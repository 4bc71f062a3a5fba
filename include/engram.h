/*
 * engram.h -- C ABI of the MI355X (gfx950) Engram conditional-memory forward
 * pass: hashed suffix n-gram embeddings fused into a hidden state by a
 * context-aware gate, a short depthwise causal convolution and a residual.
 *
 * Source pages (summaries of "Conditional Memory via Scalable Lookup: A New
 * Axis of Sparsity for Large Language Models"):
 *   [club]  discuss.deepseek.club/t/topic/717, section 二 核心创新:
 *           1.(1) 基于 N-gram 的稀疏哈希检索 (retrieval),
 *           1.(2) 上下文感知的门控机制 (fusion), 2. 工程优化 (multi-branch,
 *           prefetch), 三.4 系统效率 (throughput context)
 *   [csdn]  gitcode.csdn.net "DeepSeek又搞了个大动作，这次是真的狠",
 *           section Engram 到底怎么工作的 (four steps; layers 2 and 6)
 *   [rep]   reportify.cn tag page 条件记忆, summaries 技术方案：Engram架构,
 *           技术创新与架构 / 系统效率与扩展性 (retrieval depends only on tokens)
 *
 * Conventions (every entry point):
 *   - Pointers named d_* are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains caller memory; a plan owns only a
 *     small host struct.
 *   - Arguments are validated synchronously.  On any failure a non-zero
 *     engram_status is returned and nothing is enqueued.  Kernel launch
 *     failures return ENGRAM_E_DEVICE.  No C++ exception crosses the ABI.
 *   - Work is enqueued on the caller's stream in order; no call synchronises
 *     the stream or the device.  Calls on different streams with disjoint
 *     outputs may run concurrently; plans are immutable after creation.
 *   - Device pointers must be 16-byte aligned.
 *   - Data errors inside kernels are defined, not trapped: raw token ids
 *     outside [0, vocab) are treated as the PAD id and counted.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define ENGRAM_API __attribute__((visibility("default")))
#else
#define ENGRAM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ENGRAM_OK = 0,
    ENGRAM_E_INVALID_ARG = 1, /* null pointer, bad size, misalignment, short workspace */
    ENGRAM_E_UNSUPPORTED = 2, /* a shape the library's kernels do not cover */
    ENGRAM_E_DEVICE = 3,      /* a HIP runtime call or kernel launch failed */
    ENGRAM_E_NOMEM = 4        /* host allocation of the plan failed */
} engram_status;

typedef enum { ENGRAM_F32 = 0, ENGRAM_BF16 = 1 } engram_dtype;

/* Conv output mode.  LINEAR: y = conv(u).  SILU_SKIP: y = u + silu(conv(u)),
 * the "adds nonlinearity" reading of [club] 1.(2). */
enum { ENGRAM_CONV_LINEAR = 0, ENGRAM_CONV_SILU_SKIP = 1 };

/* engram_gate_fuse / engram_forward flag: write y instead of h + y. */
enum { ENGRAM_OUT_DELTA = 1u << 0 };
/* engram_forward flag: retrieval inside the projection launches.  On chunks
 * shorter than K_c - 1 (decode), where W_k and W_v go through one launch on
 * 128 x 128 tiles, that launch also retrieves: each workgroup hashes the
 * n-grams of its tokens and loads its E operand straight from the table
 * rows.  On longer chunks the W_k launch and the fused W_v launch each do
 * the same for their tiles.  E never reaches memory; n_tables <= 16 and
 * d_e % 8 == 0.  Same results bit for bit.  Measured at a decode step of 256
 * sequences (four branches, d = 2560, packed weights): 11% slower per step
 * than the separate retrieval kernel (0.0820 against 0.0737 ms), whose row
 * loads all go out together; before that kernel was made so it was 1.3%
 * faster.  On prefill chunks: 5% slower at 8 x 4096
 * tokens with d = 1024, 19-25% slower at d = 2560 (random row pieces from
 * HBM outrun the operand ring).  Off by default.  Ignored where it does not
 * apply. */
enum { ENGRAM_RETRIEVE_IN_PROJECTION = 1u << 1 };
/* engram_forward / engram_gate_fuse / engram_forward_noalloc flag: the W_k and
 * W_v pointers of the weights hold matrices packed by engram_pack_weight
 * (bf16 plans only; engram_backward takes the [d][D_e] matrices and rejects
 * the flag).  Same results bit for bit. */
enum { ENGRAM_WEIGHTS_PACKED = 1u << 2 };

#define ENGRAM_MAX_TABLES 32
#define ENGRAM_MAX_BRANCHES 4

typedef struct engram_plan_s *engram_plan;

typedef struct {
    int32_t vocab;       /* raw vocabulary size V                                */
    int32_t vocab_comp;  /* compressed vocabulary V' (< 2^21); PAD id = V'      */
    int32_t n_orders;    /* 1 or 2                                              */
    int32_t orders[4];   /* n-gram orders, each 2 or 3 ([csdn]: last 2 and 3)   */
    int32_t heads;       /* K hash heads per order ([club] 1.(1))               */
    int32_t head_dim;    /* d_e: row width of every table                       */
    uint32_t table_rows[ENGRAM_MAX_TABLES]; /* rows of table tau = o*K + k (primes) */
    uint64_t hash_seed;  /* seed of the per-table hash seeds                    */
    int32_t d_model;     /* hidden size d                                       */
    int32_t n_branches;  /* residual branches B_r sharing tables and W_v (1..4) */
    int32_t conv_kernel; /* depthwise causal conv taps K_c (1..4)               */
    int32_t conv_mode;   /* ENGRAM_CONV_LINEAR or ENGRAM_CONV_SILU_SKIP         */
    float rms_eps;       /* epsilon inside both RMSNorms (e.g. 1e-6)            */
    engram_dtype dtype;  /* dtype of tables, E, h, W_k, W_v and out             */
    engram_dtype state_dtype; /* element type of the carried conv state: ENGRAM_F32
                            (0, the default of a zeroed struct) or ENGRAM_BF16
                            (bf16 plans only): the gated values a chunk carries
                            are rounded to nearest-even bf16, which halves the
                            state's traffic at decode; chunked calls then agree
                            with one whole call within the bf16 tolerance
                            rather than bit for bit                          */
} engram_config;

/* Device pointers to one layer's weights; all caller-owned and read-only.
 * Multi-branch integration ([club] 2. 工程优化): branches share the tables and
 * W_v, each has its own W_k.  Conv taps are shared by all branches. */
typedef struct {
    const void *w_k[ENGRAM_MAX_BRANCHES];       /* [d][D_e] per branch, dtype; row n gives channel n */
    const void *w_v;                            /* [d][D_e], dtype                          */
    const float *gamma_h[ENGRAM_MAX_BRANCHES];  /* [d] RMSNorm weight of h, per branch      */
    const float *gamma_k[ENGRAM_MAX_BRANCHES];  /* [d] RMSNorm weight of k, per branch      */
    const float *conv_w;                        /* [d][K_c]; tap K_c-1 multiplies the current token */
} engram_weights;

/* Per-kernel timing gathered while profiling is on (see engram_profile_*). */
enum {
    ENGRAM_K_HASH = 0,    /* engram_hash                                                     */
    ENGRAM_K_GATHER = 1,  /* engram_gather, or the fused hash + gather of engram_forward      */
    ENGRAM_K_GEMM = 2,    /* projections W_k e of every branch with the gate partials fused
                             (and W_v e on the fusion-kernel path)                           */
    ENGRAM_K_FUSE = 3,    /* fusion-kernel path (short chunks, fp32): gated value, conv,
                             residual, state                                                 */
    ENGRAM_K_AUX = 4,     /* context / state bookkeeping                                      */
    ENGRAM_K_GEMM_V = 5,  /* W_v e with gated value, conv, residual, state fused (prefill)     */
    ENGRAM_K_GATE = 6,    /* gate per token and branch from the partial sums                  */
    ENGRAM_K_SEAM = 7,    /* rows at 256-token tile seams left by ENGRAM_K_GEMM_V             */
    ENGRAM_K_BWD_GEMM = 8,  /* engram_backward: the MFMA contractions (k and v again, dE, dW)  */
    ENGRAM_K_BWD_FUSE = 9,  /* engram_backward: gate statistics, conv / gate / RMSNorm backward,
                               transposes and the reductions of the small gradients           */
    ENGRAM_K_BWD_TABLE = 10,/* engram_backward: sort, scan and per-row sums of the table gradient */
    ENGRAM_K_COUNT = 11
};

typedef struct {
    double total_ms[ENGRAM_K_COUNT];
    int64_t launches[ENGRAM_K_COUNT];
    int64_t dropped; /* launches not timed because the event pool ran out */
} engram_profile;

/* Create a plan from a config (host only, no device work).  Validates the
 * config: V' < 2^21 so n-gram keys stay injective in 64 bits, n_tables =
 * n_orders*heads <= 32, every table_rows in [1, 2^31), head_dim*elem_bytes a
 * multiple of 16, 1 <= n_branches <= 4, 1 <= conv_kernel <= 4. */
ENGRAM_API engram_status engram_plan_create(const engram_config *cfg, engram_plan *out);
ENGRAM_API engram_status engram_plan_destroy(engram_plan p);

/* Bytes of device workspace engram_forward needs for batch*seqlen tokens
 * (also enough for engram_gate_fuse).  0 on invalid arguments. */
ENGRAM_API size_t engram_workspace_size(engram_plan p, int32_t batch, int32_t seqlen);

/* Pack one weight matrix (a W_k^(m) or W_v, [d][D_e] bf16, row n = channel n)
 * into the operand layout the projection kernels copy into LDS: blocks of 16
 * rows x 32 values (1 KB), block (n/16, k/32) at byte ((n/16) * D_e/32 + k/32)
 * * 1024, row n%16 of a block 64 bytes long, its four 16-byte pieces q (values
 * k%32 = 8q .. 8q+7) at positions q ^ (((r >> 1) ^ (r >> 2)) & 3) for r = n%16.
 * A ring stage then fetches each block with one linear 1 KB read instead of 16
 * rows x 64 bytes of a [d][D_e] matrix, which keeps fewer DRAM pages and cache
 * lines open per read; it is this library's own layout, not the method's
 * (measured on one MI355X, alternating runs: the 32,768-token d = 2560 layer
 * on 200 GB of tables 2% faster per step, W_k 195 -> 192 us; the four-branch
 * decode step of 256 sequences 4% faster, its projection 19.1 -> 17.2 us).
 *   d_w       [d_model][D_e] bf16 device matrix (16-byte aligned)
 *   d_packed  d_model * D_e * 2 bytes of device memory (16-byte aligned),
 *             caller-owned, not overlapping d_w; written on `stream`
 * Pass the packed matrices in engram_weights together with
 * ENGRAM_WEIGHTS_PACKED.  Packing is done once per set of weights; the
 * forward never reads the [d][D_e] form when the flag is given.
 * Errors: ENGRAM_E_INVALID_ARG (null or misaligned pointers, overlap),
 * ENGRAM_E_UNSUPPORTED (fp32 plans, shapes engram_forward rejects),
 * ENGRAM_E_DEVICE (launch failure). */
ENGRAM_API engram_status engram_pack_weight(engram_plan p, const void *d_w, void *d_packed, hipStream_t stream);

ENGRAM_API const char *engram_status_string(engram_status s);

/*
 * Retrieval, steps 1-3 ([club] 1.(1); [csdn] first two steps; [rep]
 * 技术创新与架构): compress every raw id through the vocabulary projection,
 * form the suffix n-grams of each order at every position (oldest id first;
 * positions before the sequence start take d_prev_ctx, else PAD = V'), and
 * hash each n-gram with each head into its prime-sized table.
 *   d_tokens     [batch][seqlen] int32 raw ids
 *   d_comp_map   [V] int32, values in [0, V')
 *   d_prev_ctx   [batch][2] int32 compressed ids preceding token 0 (oldest
 *                first), or NULL for a sequence start.  Not modified.
 *   d_idx        [batch*seqlen][n_tables] uint32 output slots
 *   d_bad_tokens optional uint32 counter, incremented (atomically) once per
 *                raw id outside [0, V); such ids hash as PAD.
 * The slot of an n-gram g = (g_0..g_{n-1}) in table tau is
 *   mix64(key(g) XOR s_tau) mod rows_tau,  key(g) = sum_i g_i (V'+1)^(n-1-i),
 * mix64 the SplitMix64 output function, s_tau = mix64(hash_seed +
 * (tau+1)*0x9E3779B97F4A7C15) (the pages only say the hashing is
 * deterministic and multi-headed; these constants are this library's).
 */
ENGRAM_API engram_status engram_hash(engram_plan p, const int32_t *d_tokens, int32_t batch, int32_t seqlen,
                          const int32_t *d_comp_map, const int32_t *d_prev_ctx, uint32_t *d_idx,
                          uint32_t *d_bad_tokens, hipStream_t stream);

/*
 * Retrieval, step 4 ([club] 1.(1): concatenate the heads' lookups): for every
 * token t and table tau, copy row d_idx[t][tau] of table tau into
 * E[t][tau*d_e : (tau+1)*d_e].  Bit-exact copy.
 *   d_idx       [n_tokens][n_tables] uint32, each < table_rows[tau]
 *               (larger values are clamped to the last row, never read out of bounds)
 *   table_ptrs  HOST array of n_tables DEVICE pointers, table tau is
 *               [table_rows[tau]][d_e] row-major in the plan dtype
 *   d_emb       [n_tokens][n_tables*d_e] plan dtype
 */
ENGRAM_API engram_status engram_gather(engram_plan p, const uint32_t *d_idx, int64_t n_tokens,
                            const void *const *table_ptrs, void *d_emb, hipStream_t stream);

/*
 * Tables in host memory ([rep] 工程实现与硬件效率: the pages' deployment keeps
 * the tables in host DRAM and fetches a step's rows over the host link ahead
 * of the layer, since the indices depend only on the tokens; [rep] 技术方案:
 * a multi-level cache, because n-gram accesses are Zipfian).
 *
 * engram_host_alloc returns `bytes` of pinned host memory that every GPU can
 * read directly (mapped, and cacheable by the GPU: contents must not change
 * while kernels read them).  Tables placed there are passed to engram_gather,
 * engram_gather_cached or engram_forward like device tables; each row read
 * then crosses the host link.  *ptr is set to NULL and ENGRAM_E_NOMEM returned
 * when the allocation fails.  engram_host_free releases such memory (NULL is
 * accepted); the caller makes sure no kernel still reads it.
 */
ENGRAM_API engram_status engram_host_alloc(size_t bytes, void **ptr);
ENGRAM_API engram_status engram_host_free(void *ptr);

/* A per-table cache of hot rows in device memory: open addressing over
 * `capacity` slots per table (linear probing from a multiplicative hash of
 * the row number).  All pointers are caller-owned device memory. */
typedef struct {
    uint32_t *keys;     /* [n_tables][capacity]: row + 1 of the row in each slot, 0 = free */
    void *rows;         /* [n_tables][capacity][d_e] plan dtype: copies of those rows      */
    uint32_t capacity;  /* slots per table, a power of two; 0 = no cache                   */
} engram_row_cache;

/*
 * Fill `cache` with rows d_hot[tau][0..n_hot) of every table tau, copied from
 * table_ptrs (host or device tables).  Entries >= table_rows[tau] are
 * skipped, repeated entries stored once.  Requires 2 * n_hot <= capacity (the
 * load factor stays at most 1/2, so every lookup ends within a few probes),
 * 16-byte aligned keys and rows.  Which rows are hot is the caller's choice
 * (e.g. the most frequent slots of a sample of traffic).  Slot placement may
 * differ between builds; what a lookup returns does not.
 */
ENGRAM_API engram_status engram_cache_build(engram_plan p, const uint32_t *d_hot, int32_t n_hot,
                                            const void *const *table_ptrs, const engram_row_cache *cache,
                                            hipStream_t stream);

/*
 * engram_gather with the rows found in `cache` read from it instead of the
 * tables (NULL cache or capacity 0: every row from the tables).  The result
 * is bit-identical to engram_gather on the same tables, provided the cache
 * was built from them.  max_workgroups > 0 caps the launch at that many
 * workgroups, each looping over its share of the tokens: a prefetch issued
 * on its own stream beside a model's other kernels then keeps the CU slots
 * it holds from start to end, instead of queueing one short workgroup per
 * 1024/n_tables tokens behind them (the host link needs few CUs to stay busy).
 * 0: one workgroup per 1024/n_tables tokens.  Other arguments as engram_gather.
 */
ENGRAM_API engram_status engram_gather_cached(engram_plan p, const uint32_t *d_idx, int64_t n_tokens,
                                              const void *const *table_ptrs, const engram_row_cache *cache,
                                              void *d_emb, int32_t max_workgroups, hipStream_t stream);

/*
 * Host-gather prefetch: the pages' deployment of host-resident tables ([rep]
 * 工程实现与硬件效率: the rows of a step are fetched from host DRAM while
 * earlier layers compute, since the indices depend only on the tokens).
 * Host threads look every (token, table) pair up in the HBM cache's keys and
 * copy the rows that miss into pinned staging; a DMA engine copies the
 * indices in and the staged rows out.  Until E is assembled the prefetch
 * queues no kernel, so it never waits for compute units behind the model's
 * kernels.
 *
 * engram_prefetcher_create: host_tables are HOST pointers (any host memory:
 * the host threads read them, the GPU never does), `cache` an optional
 * hot-row cache built from the same tables and left unchanged while the
 * prefetcher lives (its keys are copied to the host here; NULL: every row
 * comes from the host).  The prefetcher owns n_threads host threads
 * (1..256), a copy stream at the default priority, and staging for
 * max_tokens tokens: 2 * max_tokens * n_tables * (4 + d_e * elem) bytes of
 * device memory and max_tokens * n_tables * (8 + d_e * elem) bytes of pinned
 * host memory.  Synchronous.
 *
 * engram_prefetch_begin: once the work queued so far on `stream` is done
 * (so the indices may come from a kernel on it), d_idx [n_tok][n_tables]
 * (n_tok <= max_tokens) is copied to the host and the host threads start.
 * Returns at once.  d_idx must stay unchanged until finish returns.  One job
 * at a time: a second begin before finish returns ENGRAM_E_INVALID_ARG.
 *
 * engram_prefetch_finish blocks the calling host thread until the job's
 * rows are staged and their copy to the GPU is enqueued, then makes `stream`
 * wait for that copy and enqueues the assembly of d_emb [n_tok][n_tables*d_e]
 * (bit-identical to engram_gather on the same tables).  *h_misses_out (if
 * not NULL) receives the number of (token, table) pairs that missed the cache.
 *
 * engram_prefetcher_destroy waits for a job in flight, then releases
 * everything the prefetcher owns.
 */
typedef struct engram_prefetcher_s *engram_prefetcher;
ENGRAM_API engram_status engram_prefetcher_create(engram_plan p, const void *const *host_tables,
                                                  const engram_row_cache *cache, int64_t max_tokens,
                                                  int32_t n_threads, engram_prefetcher *out);
ENGRAM_API engram_status engram_prefetcher_destroy(engram_prefetcher f);
ENGRAM_API engram_status engram_prefetch_begin(engram_prefetcher f, const uint32_t *d_idx, int64_t n_tok,
                                               hipStream_t stream);
ENGRAM_API engram_status engram_prefetch_finish(engram_prefetcher f, void *d_emb, uint32_t *h_misses_out,
                                                hipStream_t stream);

/*
 * Fusion ([club] 1.(2); [csdn] third and fourth steps), per branch m and token t:
 *   k = W_k^(m) e_t, v = W_v e_t                      (fp32 accumulation)
 *   alpha = sigmoid( <RMSNorm_{gamma_h}(h_t), RMSNorm_{gamma_k}(k)> / sqrt(d) )
 *   u_t = alpha * v
 *   conv_t[i] = sum_j conv_w[i][K_c-1-j] * u_{t-j}[i]   (depthwise, causal)
 *   y = conv (LINEAR) or u + conv*sigmoid(conv) (SILU_SKIP)
 *   out_t = h_t + y   (or y with ENGRAM_OUT_DELTA)
 * with RMSNorm_g(x) = g * x / sqrt(mean(x^2) + eps).
 *   d_emb        [batch*seqlen][D_e], D_e = n_tables*d_e
 *   d_h, d_out   [n_branches][batch*seqlen][d]; d_out may alias d_h
 *   d_conv_state [n_branches][batch][K_c-1][d] gated values preceding
 *                position 0 (oldest first), fp32 or bf16 as the plan's
 *                state_dtype says, or NULL for zeros.  When given it is
 *                replaced by the last K_c-1 gated values of the sequence
 *                extended by this chunk, so chunked prefill and decode equal
 *                one full prefill (bit for bit with an fp32 state).
 *   d_alpha      optional [n_branches][batch*seqlen] fp32 gate values
 *   flags        ENGRAM_OUT_DELTA, ENGRAM_WEIGHTS_PACKED (W_k and W_v of w as
 *                engram_pack_weight wrote them)
 *   d_workspace  >= engram_workspace_size(p, batch, seqlen) bytes, 256-byte aligned
 * Supported: bf16 with d % 256 == 0, D_e % 128 == 0 and one branch of h
 * (batch*seqlen*d*2 bytes) under 4 GiB; f32 any d, D_e.  batch*seqlen*D_e and
 * d*D_e elements must stay under 2^31 bytes.  Anything else returns
 * ENGRAM_E_UNSUPPORTED and launches nothing.
 */
ENGRAM_API engram_status engram_gate_fuse(engram_plan p, const void *d_emb, const void *d_h, int32_t batch,
                               int32_t seqlen, const engram_weights *w, void *d_conv_state,
                               void *d_out, float *d_alpha, uint32_t flags, void *d_workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * The whole forward pass: engram_hash, engram_gather and engram_gate_fuse in
 * one call (indices and E live in the workspace).  If d_prev_ctx is non-NULL
 * it is read as in engram_hash and then replaced by the last two compressed
 * ids of the sequence extended by this chunk.  flags: those of
 * engram_gate_fuse and ENGRAM_RETRIEVE_IN_PROJECTION.
 */
ENGRAM_API engram_status engram_forward(engram_plan p, const int32_t *d_tokens, int32_t batch, int32_t seqlen,
                             const int32_t *d_comp_map, int32_t *d_prev_ctx,
                             const void *const *table_ptrs, const void *d_h,
                             const engram_weights *w, void *d_conv_state, void *d_out,
                             float *d_alpha, uint32_t flags, void *d_workspace,
                             size_t workspace_bytes, uint32_t *d_bad_tokens, hipStream_t stream);

/*
 * Retrieval on its own, ahead of the layer that uses it ([rep]
 * 工程实现与硬件效率: the slots depend only on the token ids, so a later
 * layer's rows can be fetched while earlier layers still compute).  Hashes
 * every (token, table) pair and copies its row into d_emb in one launch, as
 * engram_forward does (steps 1-4 of engram_hash and engram_gather); then, if
 * d_prev_ctx is non-NULL, replaces it by the last two compressed ids of the
 * sequence extended by this chunk (inside that launch when seqlen == 1, else a
 * second launch, one thread per sequence).
 * engram_retrieve followed by engram_gate_fuse on d_emb, on one stream or with
 * d_emb handed over between streams by an event, gives engram_forward's
 * results bit for bit.
 *   d_tokens, d_comp_map, d_prev_ctx, d_bad_tokens  as engram_forward
 *   table_ptrs   HOST array of n_tables DEVICE (or engram_host_alloc) pointers
 *   d_emb        [batch*seqlen][n_tables*d_e] plan dtype, 16-byte aligned,
 *                caller-owned; fully overwritten
 * Bad arguments return ENGRAM_E_INVALID_ARG (batch*seqlen above 2^31-1:
 * ENGRAM_E_UNSUPPORTED) and launch nothing.
 */
ENGRAM_API engram_status engram_retrieve(engram_plan p, const int32_t *d_tokens, int32_t batch, int32_t seqlen,
                              const int32_t *d_comp_map, int32_t *d_prev_ctx,
                              const void *const *table_ptrs, void *d_emb, uint32_t *d_bad_tokens,
                              hipStream_t stream);

/*
 * engram_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results (bit for bit) as engram_forward, minus the
 * workspace: the library keeps one scratch array of
 * ENGRAM_NOALLOC_SCRATCH_BYTES on each GPU it runs on (a device variable of
 * the library's code object, held until the process ends) and runs
 * engram_forward's kernels on it.  The call allocates and frees nothing; its
 * first call on a device looks the array's address up once.
 *   - A call whose engram_workspace_size(p, batch, seqlen) exceeds
 *     ENGRAM_NOALLOC_SCRATCH_BYTES returns ENGRAM_E_UNSUPPORTED and launches
 *     nothing (64 MiB covers, for example, 256 one-token sequences of four
 *     branches at d = 2560, or a 4096-token chunk at d = 2560 with 16 tables
 *     of 80 dims).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on the same GPU (other streams, other host threads) race and give
 *     wrong results.  The caller serialises them, for instance by issuing them
 *     all on one stream.  Calls on different GPUs do not interact.
 *   - ENGRAM_E_DEVICE if the runtime cannot give the array's address.
 */
#define ENGRAM_NOALLOC_SCRATCH_BYTES (64u << 20)
ENGRAM_API engram_status engram_forward_noalloc(engram_plan p, const int32_t *d_tokens, int32_t batch,
                                                int32_t seqlen, const int32_t *d_comp_map, int32_t *d_prev_ctx,
                                                const void *const *table_ptrs, const void *d_h,
                                                const engram_weights *w, void *d_conv_state, void *d_out,
                                                float *d_alpha, uint32_t flags, uint32_t *d_bad_tokens,
                                                hipStream_t stream);

/* Gradients written by engram_backward (fp32, caller-owned device memory,
 * overwritten). */
typedef struct {
    float *dw;           /* [n_branches + 1][d][D_e]: dL/dW_k of each branch, then dL/dW_v  */
    float *dgamma_h;     /* [n_branches][d]                                                 */
    float *dgamma_k;     /* [n_branches][d]                                                 */
    float *dconv_w;      /* [d][K_c]                                                        */
    uint32_t *row_ids;   /* [n_tables][batch*seqlen]: the rows of table tau that the chunk
                            gathered, distinct, ascending (the first row_counts[tau] entries) */
    float *row_grads;    /* [n_tables][batch*seqlen][d_e]: dL/d(row) of each listed row, the
                            sum over the tokens that gathered it                            */
    int32_t *row_counts; /* [n_tables]                                                      */
} engram_grads;

/* Bytes of device workspace engram_backward needs for batch*seqlen tokens
 * (0 on invalid arguments or an unsupported shape). */
ENGRAM_API size_t engram_backward_workspace_size(engram_plan p, int32_t batch, int32_t seqlen);

/*
 * Backward of engram_forward for whole sequences (no carried context or conv
 * state), for training ([csdn] 实际效果到底有多好: the slots become meaningful
 * through the gradients that reach them).  Given dL/dout, the chain rule
 * through the residual, the conv, the gated value, the sigmoid gate, both
 * RMSNorms and the projections, and the table rows each token gathered:
 *   d_idx       [batch*seqlen][n_tables] slots from engram_hash of the same tokens
 *   table_ptrs  as engram_gather (HOST array of DEVICE pointers)
 *   d_h, w      the forward's hidden state and weights
 *   d_dout      [n_branches][batch*seqlen][d] dL/dout, plan dtype
 *   flags       ENGRAM_OUT_DELTA if the forward wrote y (then dout reaches h
 *               only through the gate); w holds [d][D_e] matrices
 *               (ENGRAM_WEIGHTS_PACKED is rejected)
 *   d_dh        [n_branches][batch*seqlen][d] dL/dh, plan dtype (out)
 *   g           the other gradients (out)
 * Every table row's gradient is the sum over the tokens that gathered it,
 * added in token order: the result does not depend on scheduling.
 * Supported: bf16 plans with d % 256 == 0 and D_e % 128 == 0 (the forward's
 * MFMA shapes); anything else returns ENGRAM_E_UNSUPPORTED.
 */
ENGRAM_API engram_status engram_backward(engram_plan p, const uint32_t *d_idx, const void *const *table_ptrs,
                              const void *d_h, const engram_weights *w, const void *d_dout,
                              int32_t batch, int32_t seqlen, uint32_t flags, void *d_dh,
                              const engram_grads *g, void *d_workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Profiling: while on, each launch of a kind selected by kind_mask (bit k
 * selects ENGRAM_K_* value k; 0 selects every kind) is timed by a pair of HIP
 * events that the kernel's own dispatch records (hipExtLaunchKernel), on the
 * launch stream, at most max_launches launches.  Launches of other kinds run
 * untimed.  engram_profile_end synchronises on those events, fills *out with
 * per-kind totals and turns profiling off.  Not thread-safe per plan.
 */
ENGRAM_API engram_status engram_profile_begin(engram_plan p, int32_t max_launches, uint32_t kind_mask);
ENGRAM_API engram_status engram_profile_end(engram_plan p, engram_profile *out);
/*
 * Sampling for the profiling above: from the next engram_profile_begin on,
 * only the first launch of every `every` launches of each selected kind is
 * timed (1, the default, times them all), so that timing a kind inside a
 * measured loop adds its event overhead to one launch in `every`.  The
 * setting stays until changed.  ENGRAM_E_INVALID_ARG for every < 1.
 */
ENGRAM_API engram_status engram_profile_every(engram_plan p, int32_t every);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
