/*
 * engram_oracle.c -- plain, slow, single-threaded CPU oracle for the Engram
 * conditional-memory forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and the two
 * share no code, headers, tables or constant generators.
 *
 * Sources (the five web pages summarising "Conditional Memory via Scalable
 * Lookup: A New Axis of Sparsity for Large Language Models"):
 *   [club]     discuss.deepseek.club/t/topic/717, section 二 "核心创新":
 *              1.(1) 基于 N-gram 的稀疏哈希检索, 1.(2) 上下文感知的门控机制,
 *              2. 工程优化 (multi-branch integration)
 *   [csdn]     gitcode.csdn.net article "DeepSeek又搞了个大动作，这次是真的狠",
 *              section "Engram 到底怎么工作的"
 *   [sechub]   sechub.in/view/3162389 (answer on the Engram retrieval design)
 *   [reportify] reportify.cn tag page 条件记忆, summaries "技术方案：Engram架构",
 *              "技术创新与架构", "技术原理与设计"
 * The pages describe the method in words only; where they leave a step open
 * (hash function, table sizes, padding, conv form, gate constants) this file
 * takes the readings listed in the design notes, each marked "reading:".
 *
 * Everything floating point is accumulated in double.  bf16/fp32 inputs are
 * widened exactly on read.  Build: gcc -O2 -ffp-contract=off -fPIC -shared.
 *
 * Parity status: every function here is pinned by CPU tests (known-answer
 * values of the published generators, brute force over tiny vocabularies,
 * closed forms of the gate, a library depthwise convolution, NumPy fp64
 * matmul).  End-to-end equality with DeepSeek's own Engram is parity
 * unpinned: no code, weights or printed values exist to compare against.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_CONV_LINEAR 0
#define ORC_CONV_SILU_SKIP 1
#define ORC_OUT_DELTA 1u

/* ------------------------------------------------------------------------ */
/* element access                                                           */
/* ------------------------------------------------------------------------ */

static double orc_bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Read element i of an array stored as fp32 or bf16, widened exactly. */
static double orc_load(const void *p, int64_t i, int dtype) {
    if (dtype == ORC_BF16) return orc_bf16_to_double(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t orc_bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* O3 building blocks: the 64-bit mixer and per-table seeds                 */
/* ------------------------------------------------------------------------ */

/* reading: the pages only say the hashing is deterministic and multi-head
 * ([club] 1.(1); [reportify] 技术方案).  The mixer is the SplitMix64 output
 * function (Steele, Lea & Flood, OOPSLA 2014, with Stafford's Mix13
 * constants), a bijection on 64-bit words. */
uint64_t orc_mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

/* The tau-th output of a SplitMix64 stream seeded with hash_seed: every
 * table (hash head) gets its own independent 64-bit seed. */
uint64_t orc_table_seed(uint64_t hash_seed, int32_t tau) {
    uint64_t state = hash_seed + (uint64_t)(tau + 1) * 0x9E3779B97F4A7C15ull;
    return orc_mix64(state);
}

/* Key of an n-gram and its slot in one table.  g[0..n-1] are compressed ids, oldest
 * first, each in [0, vocab_comp] (vocab_comp itself is the PAD id used before
 * the start of a sequence).  The n-gram is packed injectively as a base
 * (vocab_comp+1) number, mixed with the table's seed and reduced modulo the
 * table's prime row count. */
uint64_t orc_ngram_key(const int32_t *g, int32_t n, int32_t vocab_comp) {
    uint64_t base = (uint64_t)vocab_comp + 1u;
    uint64_t key = 0;
    for (int32_t i = 0; i < n; ++i) key = key * base + (uint64_t)g[i];
    return key;
}

uint32_t orc_ngram_slot(const int32_t *g, int32_t n, int32_t vocab_comp,
                        uint64_t seed_tau, uint32_t prime) {
    uint64_t z = orc_mix64(orc_ngram_key(g, n, vocab_comp) ^ seed_tau);
    return (uint32_t)(z % (uint64_t)prime);
}

/* ------------------------------------------------------------------------ */
/* O1-O3: compression, suffix n-grams, multi-head hashing                   */
/* ------------------------------------------------------------------------ */

/* Compressed id of one raw token: the vocabulary projection maps
 * surface variants to one id ([club] 1.(1) 词汇投影; [reportify] about 23%
 * fewer ids).  Raw ids outside [0, vocab) become PAD (reading). */
static int32_t orc_compress_one(int32_t x, const int32_t *comp_map, int32_t vocab,
                                int32_t vocab_comp, int64_t *bad) {
    if (x < 0 || x >= vocab) {
        if (bad) (*bad)++;
        return vocab_comp;
    }
    return comp_map[x];
}

/*
 * Hash every position of every sequence.
 *   tokens   [batch][seqlen] raw ids
 *   prev_ctx [batch][2] compressed ids that precede token 0 (oldest first),
 *            or NULL: the sequence starts here and earlier positions are PAD
 *   primes   [n_orders*heads] rows of table tau = (order index)*heads + head
 *   idx      [batch*seqlen][n_orders*heads] output slots
 *   new_ctx  [batch][2] (may be NULL): the last two compressed ids of
 *            prev_ctx followed by this chunk
 * At every position t the suffix n-gram of order n is (c[t-n+1], ..., c[t])
 * ([csdn] "Engram 到底怎么工作的", first step: the last two and last three
 * tokens; [reportify] 技术创新与架构: suffix n-grams of the current position).
 * Returns the number of raw ids outside [0, vocab).
 */
int64_t orc_hash(const int32_t *tokens, int64_t batch, int64_t seqlen,
                 const int32_t *comp_map, int32_t vocab, int32_t vocab_comp,
                 const int32_t *prev_ctx, int32_t n_orders, const int32_t *orders,
                 int32_t heads, const uint32_t *primes, uint64_t hash_seed,
                 uint32_t *idx, int32_t *new_ctx) {
    int64_t bad = 0;
    int32_t n_tables = n_orders * heads;
    for (int64_t b = 0; b < batch; ++b) {
        /* ext = [ctx0, ctx1, c_0, c_1, ..., c_{seqlen-1}] */
        int32_t *ext = (int32_t *)malloc(sizeof(int32_t) * (size_t)(seqlen + 2));
        ext[0] = prev_ctx ? prev_ctx[b * 2 + 0] : vocab_comp;
        ext[1] = prev_ctx ? prev_ctx[b * 2 + 1] : vocab_comp;
        for (int64_t t = 0; t < seqlen; ++t)
            ext[t + 2] = orc_compress_one(tokens[b * seqlen + t], comp_map, vocab, vocab_comp, &bad);
        for (int64_t t = 0; t < seqlen; ++t) {
            int64_t row = b * seqlen + t;
            for (int32_t o = 0; o < n_orders; ++o) {
                int32_t n = orders[o];
                int32_t g[3];
                for (int32_t i = 0; i < n; ++i) g[i] = ext[t + 2 - (n - 1) + i];
                for (int32_t k = 0; k < heads; ++k) {
                    int32_t tau = o * heads + k;
                    idx[row * n_tables + tau] =
                        orc_ngram_slot(g, n, vocab_comp, orc_table_seed(hash_seed, tau), primes[tau]);
                }
            }
        }
        if (new_ctx) {
            new_ctx[b * 2 + 0] = ext[seqlen + 0];
            new_ctx[b * 2 + 1] = ext[seqlen + 1];
        }
        free(ext);
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Synthetic table contents (harness): Philox4x64-10                         */
/* ------------------------------------------------------------------------ */

/* Philox4x64 with 10 rounds, from its published definition (Salmon, Moraes,
 * Dror & Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11). */
void orc_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        unsigned __int128 p0 = (unsigned __int128)0xD2E7470EE14C6C93ull * c0;
        unsigned __int128 p1 = (unsigned __int128)0xCA5A826395121157ull * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* fp32 value of synthetic table tau at (row, col); Irwin-Hall(4) of the
 * 16-bit fields of one Philox word, scaled to standard deviation 0.02. */
float orc_synth_value(uint64_t seed, int32_t tau, uint64_t row, int32_t col) {
    uint64_t ctr[4] = {row, (uint64_t)(col / 4), (uint64_t)tau, 0};
    uint64_t key[2] = {seed, 0};
    uint64_t w[4];
    orc_philox4x64_10(ctr, key, w);
    uint64_t x = w[col % 4];
    int32_t s = (int32_t)(x & 0xFFFF) + (int32_t)((x >> 16) & 0xFFFF) +
                (int32_t)((x >> 32) & 0xFFFF) + (int32_t)((x >> 48) & 0xFFFF);
    const float scale = 0x1.1bc77ap-21f;
    float centred = (float)(s - 131070);
    return centred * scale;
}

/* ------------------------------------------------------------------------ */
/* O4: gather and concatenate                                               */
/* ------------------------------------------------------------------------ */

/* E[t] = concat over tau of Table_tau[idx[t][tau]] ([club] 1.(1): the K heads'
 * lookups are concatenated; tables of order 2 first, then order 3).  Tables
 * are the synthetic ones above; the row is stored in the table's dtype, so
 * the output holds raw fp32 values or raw bf16 bit patterns. */
void orc_gather_synth(const uint32_t *idx, int64_t n_tok, int32_t n_tables, int32_t head_dim,
                      uint64_t table_seed, int32_t dtype, void *emb) {
    int64_t De = (int64_t)n_tables * head_dim;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int32_t tau = 0; tau < n_tables; ++tau) {
            uint64_t row = idx[t * n_tables + tau];
            for (int32_t c = 0; c < head_dim; ++c) {
                float v = orc_synth_value(table_seed, tau, row, c);
                int64_t o = t * De + (int64_t)tau * head_dim + c;
                if (dtype == ORC_BF16) ((uint16_t *)emb)[o] = orc_bf16_rne(v);
                else ((float *)emb)[o] = v;
            }
        }
}

/* Same, from tables held in host memory: tables[tau] is [rows][head_dim]. */
void orc_gather_host(const uint32_t *idx, int64_t n_tok, int32_t n_tables, int32_t head_dim,
                     const void *const *tables, int32_t dtype, void *emb) {
    int64_t De = (int64_t)n_tables * head_dim;
    size_t es = dtype == ORC_BF16 ? 2 : 4;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int32_t tau = 0; tau < n_tables; ++tau) {
            const char *src = (const char *)tables[tau] + (size_t)idx[t * n_tables + tau] * head_dim * es;
            char *dst = (char *)emb + ((size_t)t * De + (size_t)tau * head_dim) * es;
            memcpy(dst, src, head_dim * es);
        }
}

/* ------------------------------------------------------------------------ */
/* O5-O7: projections, context-aware gate, gated value                       */
/* ------------------------------------------------------------------------ */

/*
 * Gate and gated value of one token for one branch.
 *   e        [De] gathered embedding (dtype)
 *   h        [d]  hidden state of this branch at this token (dtype)
 *   w_k, w_v [d][De] (row n produces output channel n) (dtype)
 *   gamma_h, gamma_k [d] fp32 RMSNorm weights
 * The hidden state acts as the query and the retrieved embedding as key and
 * value through learned projections ([club] 1.(2)); the gate is a scalar per
 * token that shrinks as key and query disagree ([club] 1.(2): alpha_t).
 * reading: alpha = sigmoid(<RMSNorm(h), RMSNorm(W_k e)> / sqrt(d)), RMSNorm
 * with weights gamma and eps inside the root, u = alpha * (W_v e).
 * Outputs alpha and u[d] (may be NULL).
 */
/* y = W e for one token: W is [d][De] (row n produces channel n). */
void orc_project(const void *e, const void *w, int32_t d, int32_t De, int32_t dtype, double *y) {
    for (int32_t n = 0; n < d; ++n) {
        double acc = 0.0;
        for (int32_t j = 0; j < De; ++j)
            acc += orc_load(e, j, dtype) * orc_load(w, (int64_t)n * De + j, dtype);
        y[n] = acc;
    }
}

double orc_gate_token(const void *e, const void *h, const void *w_k, const void *w_v,
                      const float *gamma_h, const float *gamma_k, int32_t d, int32_t De,
                      double eps, int32_t dtype, double *u) {
    double *k = (double *)malloc(sizeof(double) * (size_t)d);
    orc_project(e, w_k, d, De, dtype, k);
    double sh = 0.0, sk = 0.0;
    for (int32_t n = 0; n < d; ++n) {
        double hn = orc_load(h, n, dtype);
        sh += hn * hn;
        sk += k[n] * k[n];
    }
    double rh = sqrt(sh / d + eps);
    double rk = sqrt(sk / d + eps);
    double dot = 0.0;
    for (int32_t n = 0; n < d; ++n) {
        double qn = orc_load(h, n, dtype) * (double)gamma_h[n] / rh;
        double kn = k[n] * (double)gamma_k[n] / rk;
        dot += qn * kn;
    }
    double s = dot / sqrt((double)d);
    double alpha = 1.0 / (1.0 + exp(-s));
    if (u) {
        orc_project(e, w_v, d, De, dtype, u);
        for (int32_t n = 0; n < d; ++n) u[n] = alpha * u[n];
    }
    free(k);
    return alpha;
}

/* ------------------------------------------------------------------------ */
/* O8-O10: depthwise causal conv, residual, state                            */
/* ------------------------------------------------------------------------ */

/*
 * Engram output for positions [t0, t1) of sequence b, every branch.
 *   emb        [batch*seqlen][De] (dtype), rows of sequence b are b*seqlen+t
 *   h          [n_branches][batch*seqlen][d] (dtype)
 *   w_k        [n_branches][d][De]; w_v [d][De] (dtype)
 *   gamma_h/k  [n_branches][d] fp32
 *   conv_w     [d][conv_k] fp32, tap conv_k-1 multiplies the current token
 *   conv_state [n_branches][batch][conv_k-1][d] fp32 gated values preceding
 *              position 0 (oldest first), or NULL for zeros
 *   out        [n_branches][t1-t0][d]   h + y, or y with ORC_OUT_DELTA
 *   alpha      [n_branches][t1-t0] (may be NULL)
 *   u_out      [n_branches][t1-t0][d] (may be NULL) gated values
 * The short depthwise causal conv widens the receptive field and the result
 * joins the backbone through a residual ([club] 1.(2), last bullet; [sechub]).
 * reading: conv_t = sum_j w[conv_k-1-j] * u_{t-j}; LINEAR y = conv, SILU_SKIP
 * y = u + conv * sigmoid(conv).
 */
int32_t orc_forward_range(int64_t b, int64_t t0, int64_t t1, int64_t batch, int64_t seqlen,
                          int32_t d, int32_t De, int32_t n_branches, int32_t conv_k,
                          int32_t conv_mode, double eps, uint32_t flags, int32_t dtype,
                          const void *emb, const void *h, const void *w_k, const void *w_v,
                          const float *gamma_h, const float *gamma_k, const float *conv_w,
                          const float *conv_state, double *out, double *alpha, double *u_out) {
    if (b < 0 || b >= batch || t0 < 0 || t1 > seqlen || t0 >= t1 || conv_k < 1) return 1;
    int64_t n_tok = batch * seqlen;
    int64_t lo = t0 - (conv_k - 1); /* first position whose u is needed */
    int64_t span = t1 - lo;
    double *u = (double *)calloc((size_t)(span * d), sizeof(double));
    double *al = (double *)calloc((size_t)span, sizeof(double));
    size_t es = dtype == ORC_BF16 ? 2 : 4;
    for (int32_t m = 0; m < n_branches; ++m) {
        const char *hm = (const char *)h + (size_t)m * n_tok * d * es;
        const char *wkm = (const char *)w_k + (size_t)m * d * De * es;
        for (int64_t p = lo; p < t1; ++p) {
            double *up = u + (p - lo) * d;
            if (p < 0) {
                int64_t j = (conv_k - 1) + p; /* state row, oldest first */
                for (int32_t n = 0; n < d; ++n)
                    up[n] = conv_state
                        ? (double)conv_state[(((int64_t)m * batch + b) * (conv_k - 1) + j) * d + n]
                        : 0.0;
                continue;
            }
            int64_t row = b * seqlen + p;
            al[p - lo] = orc_gate_token((const char *)emb + (size_t)row * De * es,
                                        hm + (size_t)row * d * es, wkm, w_v,
                                        gamma_h + (size_t)m * d, gamma_k + (size_t)m * d,
                                        d, De, eps, dtype, up);
        }
        for (int64_t t = t0; t < t1; ++t) {
            int64_t row = b * seqlen + t;
            double *ut = u + (t - lo) * d;
            for (int32_t n = 0; n < d; ++n) {
                double conv = 0.0;
                for (int32_t j = 0; j < conv_k; ++j)
                    conv += (double)conv_w[(int64_t)n * conv_k + (conv_k - 1 - j)] *
                            u[(t - j - lo) * d + n];
                double y = conv;
                if (conv_mode == ORC_CONV_SILU_SKIP) y = ut[n] + conv / (1.0 + exp(-conv));
                double hv = orc_load(hm, row * d + n, dtype);
                out[((int64_t)m * (t1 - t0) + (t - t0)) * d + n] = (flags & ORC_OUT_DELTA) ? y : hv + y;
                if (u_out) u_out[((int64_t)m * (t1 - t0) + (t - t0)) * d + n] = ut[n];
            }
            if (alpha) alpha[(int64_t)m * (t1 - t0) + (t - t0)] = al[t - lo];
        }
    }
    free(u);
    free(al);
    return 0;
}

/*
 * New conv state after a chunk: the last conv_k-1 gated values of the
 * sequence extended by this chunk (state rows first, then the chunk).
 *   u_tail [n_branches][batch][min(seqlen, conv_k-1)][d]: the chunk's last
 *          gated values, oldest first
 *   state  [n_branches][batch][conv_k-1][d] in/out (NULL input = zeros)
 */
void orc_conv_state_update(int64_t batch, int64_t seqlen, int32_t d, int32_t n_branches,
                           int32_t conv_k, const double *u_tail, const float *state_in,
                           float *state_out) {
    int32_t S = conv_k - 1;
    int64_t tail = seqlen < S ? seqlen : S;
    for (int32_t m = 0; m < n_branches; ++m)
        for (int64_t b = 0; b < batch; ++b)
            for (int32_t j = 0; j < S; ++j) {
                /* extended index of state slot j: total = S + seqlen rows,
                 * slot j takes row S + seqlen - S + j = seqlen + j */
                int64_t e = seqlen + j; /* index into [state(S) | chunk(seqlen)] */
                for (int32_t n = 0; n < d; ++n) {
                    double v;
                    if (e < S) {
                        v = state_in ? (double)state_in[(((int64_t)m * batch + b) * S + e) * d + n] : 0.0;
                    } else {
                        int64_t t = e - S;           /* chunk position */
                        int64_t k = t - (seqlen - tail); /* index into u_tail */
                        v = u_tail[(((int64_t)m * batch + b) * tail + k) * d + n];
                    }
                    state_out[(((int64_t)m * batch + b) * S + j) * d + n] = (float)v;
                }
            }
}

/* ------------------------------------------------------------------------ */
/* Backward of O5-O10 (gradients for training)                               */
/* ------------------------------------------------------------------------ */

/*
 * Gradients of L = <dout, out> for whole sequences (no carried conv state),
 * every branch.  The pages say the table slots learn from the gradients that
 * reach them ([csdn] 实际效果到底有多好); the derivative itself is the chain
 * rule through the forward of orc_forward_range, written out step by step:
 *   out = h + y (or y with ORC_OUT_DELTA)            dh += dout
 *   y = conv (LINEAR) or u + conv*sigmoid(conv)      dconv, du (direct term)
 *   conv_t = sum_j w[K-1-j] u_{t-j}                  du_t += sum_j w[K-1-j] dconv_{t+j},
 *                                                    dw[K-1-j] += sum_t u_{t-j} dconv_t
 *   u = alpha v                                      dalpha = <v, du>, dv += alpha du
 *   alpha = sigmoid(s)                               ds = dalpha alpha (1 - alpha)
 *   s = <a, b>/sqrt(d), a = gh*h/rh, b = gk*k/rk     da = ds b/sqrt(d), db = ds a/sqrt(d)
 *   RMSNorm x -> g*x/r, r = sqrt(mean(x^2) + eps)    dgamma += dy x/r,
 *                                                    dx = (g*dy - (x/r) <g*dy, x/r>/d) / r
 *   k = W_k e, v = W_v e                             dW += d(k|v) e^T, de += W^T d(k|v)
 * Inputs as orc_forward_range (dtype fp32 or bf16), dout [n_branches][n_tok][d].
 * Outputs (double, overwritten):
 *   dh [n_branches][n_tok][d], demb [n_tok][De], dw_k [n_branches][d][De],
 *   dw_v [d][De], dgamma_h/dgamma_k [n_branches][d], dconv_w [d][conv_k].
 */
int32_t orc_backward(int64_t batch, int64_t seqlen, int32_t d, int32_t De, int32_t n_branches,
                     int32_t conv_k, int32_t conv_mode, double eps, uint32_t flags, int32_t dtype,
                     const void *emb, const void *h, const void *w_k, const void *w_v,
                     const float *gamma_h, const float *gamma_k, const float *conv_w,
                     const void *dout, double *dh, double *demb, double *dw_k, double *dw_v,
                     double *dgamma_h, double *dgamma_k, double *dconv_w) {
    if (batch < 1 || seqlen < 1 || d < 1 || De < 1 || n_branches < 1 || conv_k < 1) return 1;
    const int64_t n_tok = batch * seqlen;
    const size_t es = dtype == ORC_BF16 ? 2 : 4;
    const double sqd = sqrt((double)d);
    memset(dh, 0, sizeof(double) * (size_t)(n_branches * n_tok * d));
    memset(demb, 0, sizeof(double) * (size_t)(n_tok * De));
    memset(dw_k, 0, sizeof(double) * (size_t)((int64_t)n_branches * d * De));
    memset(dw_v, 0, sizeof(double) * (size_t)((int64_t)d * De));
    memset(dgamma_h, 0, sizeof(double) * (size_t)(n_branches * d));
    memset(dgamma_k, 0, sizeof(double) * (size_t)(n_branches * d));
    memset(dconv_w, 0, sizeof(double) * (size_t)(d * conv_k));

    double *V = (double *)malloc(sizeof(double) * (size_t)(seqlen * d));   /* v of every position */
    double *DV = (double *)malloc(sizeof(double) * (size_t)(seqlen * d));  /* dv, summed over branches */
    double *Kk = (double *)malloc(sizeof(double) * (size_t)(seqlen * d));  /* k of this branch */
    double *U = (double *)malloc(sizeof(double) * (size_t)(seqlen * d));
    double *CV = (double *)malloc(sizeof(double) * (size_t)(seqlen * d));  /* conv */
    double *DC = (double *)malloc(sizeof(double) * (size_t)(seqlen * d));  /* dconv */
    double *DU = (double *)malloc(sizeof(double) * (size_t)(seqlen * d));
    double *al = (double *)malloc(sizeof(double) * (size_t)seqlen);
    double *rh = (double *)malloc(sizeof(double) * (size_t)seqlen);
    double *rk = (double *)malloc(sizeof(double) * (size_t)seqlen);
    double *dk = (double *)malloc(sizeof(double) * (size_t)d);

    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t t = 0; t < seqlen; ++t)
            orc_project((const char *)emb + (size_t)(b * seqlen + t) * De * es, w_v, d, De, dtype, V + t * d);
        memset(DV, 0, sizeof(double) * (size_t)(seqlen * d));
        for (int32_t m = 0; m < n_branches; ++m) {
            const char *hm = (const char *)h + (size_t)m * n_tok * d * es;
            const char *wkm = (const char *)w_k + (size_t)m * d * De * es;
            const char *gm = (const char *)dout + (size_t)m * n_tok * d * es;
            const float *gh = gamma_h + (size_t)m * d, *gk = gamma_k + (size_t)m * d;
            /* forward: k, the gate and the gated values */
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t row = b * seqlen + t;
                double *kt = Kk + t * d;
                orc_project((const char *)emb + (size_t)row * De * es, wkm, d, De, dtype, kt);
                double sh = 0.0, sk = 0.0;
                for (int32_t n = 0; n < d; ++n) {
                    double hn = orc_load(hm, row * d + n, dtype);
                    sh += hn * hn;
                    sk += kt[n] * kt[n];
                }
                rh[t] = sqrt(sh / d + eps);
                rk[t] = sqrt(sk / d + eps);
                double dot = 0.0;
                for (int32_t n = 0; n < d; ++n)
                    dot += (orc_load(hm, row * d + n, dtype) * gh[n] / rh[t]) * (kt[n] * gk[n] / rk[t]);
                al[t] = 1.0 / (1.0 + exp(-dot / sqd));
                for (int32_t n = 0; n < d; ++n) U[t * d + n] = al[t] * V[t * d + n];
            }
            for (int64_t t = 0; t < seqlen; ++t)
                for (int32_t n = 0; n < d; ++n) {
                    double c = 0.0;
                    for (int32_t j = 0; j < conv_k && j <= t; ++j)
                        c += (double)conv_w[(int64_t)n * conv_k + (conv_k - 1 - j)] * U[(t - j) * d + n];
                    CV[t * d + n] = c;
                }
            /* backward through the output, the conv and the gated value */
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t row = b * seqlen + t;
                for (int32_t n = 0; n < d; ++n) {
                    double g = orc_load(gm, row * d + n, dtype);
                    double c = CV[t * d + n];
                    double dc = g;
                    if (conv_mode == ORC_CONV_SILU_SKIP) {
                        double sg = 1.0 / (1.0 + exp(-c));
                        dc = g * (sg + c * sg * (1.0 - sg));
                    }
                    DC[t * d + n] = dc;
                    if (!(flags & ORC_OUT_DELTA)) dh[((int64_t)m * n_tok + row) * d + n] = g;
                }
            }
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t row = b * seqlen + t;
                for (int32_t n = 0; n < d; ++n) {
                    double du = conv_mode == ORC_CONV_SILU_SKIP ? orc_load(gm, row * d + n, dtype) : 0.0;
                    for (int32_t j = 0; j < conv_k && t + j < seqlen; ++j)
                        du += (double)conv_w[(int64_t)n * conv_k + (conv_k - 1 - j)] * DC[(t + j) * d + n];
                    DU[t * d + n] = du;
                    for (int32_t j = 0; j < conv_k && j <= t; ++j)
                        dconv_w[(int64_t)n * conv_k + (conv_k - 1 - j)] += U[(t - j) * d + n] * DC[t * d + n];
                }
            }
            /* backward through the gate, both RMSNorms and W_k */
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t row = b * seqlen + t;
                const double *kt = Kk + t * d;
                double dal = 0.0;
                for (int32_t n = 0; n < d; ++n) {
                    dal += V[t * d + n] * DU[t * d + n];
                    DV[t * d + n] += al[t] * DU[t * d + n];
                }
                const double ds = dal * al[t] * (1.0 - al[t]);
                double Sh = 0.0, Sk = 0.0;
                for (int32_t n = 0; n < d; ++n) {
                    const double hn = orc_load(hm, row * d + n, dtype);
                    const double an = gh[n] * hn / rh[t], bn = gk[n] * kt[n] / rk[t];
                    const double da = ds * bn / sqd, db = ds * an / sqd;
                    dgamma_h[(int64_t)m * d + n] += da * hn / rh[t];
                    dgamma_k[(int64_t)m * d + n] += db * kt[n] / rk[t];
                    Sh += gh[n] * da * (hn / rh[t]);
                    Sk += gk[n] * db * (kt[n] / rk[t]);
                }
                for (int32_t n = 0; n < d; ++n) {
                    const double hn = orc_load(hm, row * d + n, dtype);
                    const double an = gh[n] * hn / rh[t], bn = gk[n] * kt[n] / rk[t];
                    const double da = ds * bn / sqd, db = ds * an / sqd;
                    dh[((int64_t)m * n_tok + row) * d + n] += (gh[n] * da - (hn / rh[t]) * Sh / d) / rh[t];
                    dk[n] = (gk[n] * db - (kt[n] / rk[t]) * Sk / d) / rk[t];
                }
                for (int32_t n = 0; n < d; ++n)
                    for (int32_t j = 0; j < De; ++j) {
                        const double ej = orc_load((const char *)emb + (size_t)row * De * es, j, dtype);
                        dw_k[((int64_t)m * d + n) * De + j] += dk[n] * ej;
                        demb[row * De + j] += orc_load(wkm, (int64_t)n * De + j, dtype) * dk[n];
                    }
            }
        }
        /* W_v, shared by the branches */
        for (int64_t t = 0; t < seqlen; ++t) {
            const int64_t row = b * seqlen + t;
            for (int32_t n = 0; n < d; ++n)
                for (int32_t j = 0; j < De; ++j) {
                    const double ej = orc_load((const char *)emb + (size_t)row * De * es, j, dtype);
                    dw_v[(int64_t)n * De + j] += DV[t * d + n] * ej;
                    demb[row * De + j] += orc_load(w_v, (int64_t)n * De + j, dtype) * DV[t * d + n];
                }
        }
    }
    free(V); free(DV); free(Kk); free(U); free(CV); free(DC); free(DU);
    free(al); free(rh); free(rk); free(dk);
    return 0;
}

/* One (row, token) pair of a table's gathered rows, for the sort below. */
typedef struct {
    uint32_t row;
    int64_t t;
} orc_row_use;

static int orc_row_use_cmp(const void *x, const void *y) {
    const orc_row_use *a = (const orc_row_use *)x, *b = (const orc_row_use *)y;
    if (a->row != b->row) return a->row < b->row ? -1 : 1;
    return a->t < b->t ? -1 : (a->t > b->t);
}

/*
 * Gradient of the table rows a chunk gathered: token t's row of table tau,
 * idx[t][tau], receives demb[t][tau*head_dim : (tau+1)*head_dim].  Per table,
 * the distinct rows in ascending order and each row's summed gradient (added
 * in ascending token order).
 *   rows   [n_tables][n_tok]            (the first counts[tau] entries used)
 *   grads  [n_tables][n_tok][head_dim]  (likewise)
 *   counts [n_tables]
 */
void orc_table_grad(const uint32_t *idx, int64_t n_tok, int32_t n_tables, int32_t head_dim,
                    const double *demb, uint32_t *rows, double *grads, int64_t *counts) {
    const int64_t De = (int64_t)n_tables * head_dim;
    orc_row_use *use = (orc_row_use *)malloc(sizeof(orc_row_use) * (size_t)n_tok);
    for (int32_t tau = 0; tau < n_tables; ++tau) {
        for (int64_t t = 0; t < n_tok; ++t) {
            use[t].row = idx[t * n_tables + tau];
            use[t].t = t;
        }
        qsort(use, (size_t)n_tok, sizeof(orc_row_use), orc_row_use_cmp);
        int64_t r = -1;
        for (int64_t i = 0; i < n_tok; ++i) {
            if (i == 0 || use[i].row != use[i - 1].row) {
                ++r;
                rows[(int64_t)tau * n_tok + r] = use[i].row;
                for (int32_t c = 0; c < head_dim; ++c) grads[((int64_t)tau * n_tok + r) * head_dim + c] = 0.0;
            }
            for (int32_t c = 0; c < head_dim; ++c)
                grads[((int64_t)tau * n_tok + r) * head_dim + c] += demb[use[i].t * De + (int64_t)tau * head_dim + c];
        }
        counts[tau] = r + 1;
    }
    free(use);
}
