/* Runs every entry point of the CPU oracle (oracle/engram_oracle.c) once or
 * more on small inputs, each buffer allocated at exactly the size the
 * function's comment gives, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer reports any access outside them.  Shapes cover
 * both n-gram orders, a carried context and conv state, chunks shorter than
 * the conv window, every conv kernel size, both conv modes, fp32 and bf16.
 * Prints "ok" and exits 0 when every call returned its success code. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t orc_bf16_rne(float x);
uint64_t orc_mix64(uint64_t z);
uint64_t orc_table_seed(uint64_t hash_seed, int32_t tau);
uint64_t orc_ngram_key(const int32_t *g, int32_t n, int32_t vocab_comp);
uint32_t orc_ngram_slot(const int32_t *g, int32_t n, int32_t vocab_comp, uint64_t seed_tau, uint32_t prime);
int64_t orc_hash(const int32_t *tokens, int64_t batch, int64_t seqlen, const int32_t *comp_map, int32_t vocab,
                 int32_t vocab_comp, const int32_t *prev_ctx, int32_t n_orders, const int32_t *orders, int32_t heads,
                 const uint32_t *primes, uint64_t hash_seed, uint32_t *idx, int32_t *new_ctx);
void orc_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]);
float orc_synth_value(uint64_t seed, int32_t tau, uint64_t row, int32_t col);
void orc_gather_synth(const uint32_t *idx, int64_t n_tok, int32_t n_tables, int32_t head_dim, uint64_t table_seed,
                      int32_t dtype, void *emb);
void orc_gather_host(const uint32_t *idx, int64_t n_tok, int32_t n_tables, int32_t head_dim,
                     const void *const *tables, int32_t dtype, void *emb);
void orc_project(const void *e, const void *w, int32_t d, int32_t De, int32_t dtype, double *y);
double orc_gate_token(const void *e, const void *h, const void *w_k, const void *w_v, const float *gamma_h,
                      const float *gamma_k, int32_t d, int32_t De, double eps, int32_t dtype, double *u);
int32_t orc_forward_range(int64_t b, int64_t t0, int64_t t1, int64_t batch, int64_t seqlen, int32_t d, int32_t De,
                          int32_t n_branches, int32_t conv_k, int32_t conv_mode, double eps, uint32_t flags,
                          int32_t dtype, const void *emb, const void *h, const void *w_k, const void *w_v,
                          const float *gamma_h, const float *gamma_k, const float *conv_w, const float *conv_state,
                          double *out, double *alpha, double *u_out);
void orc_conv_state_update(int64_t batch, int64_t seqlen, int32_t d, int32_t n_branches, int32_t conv_k,
                           const double *u_tail, const float *state_in, float *state_out);
int32_t orc_backward(int64_t batch, int64_t seqlen, int32_t d, int32_t De, int32_t n_branches, int32_t conv_k,
                     int32_t conv_mode, double eps, uint32_t flags, int32_t dtype, const void *emb, const void *h,
                     const void *w_k, const void *w_v, const float *gamma_h, const float *gamma_k,
                     const float *conv_w, const void *dout, double *dh, double *demb, double *dw_k, double *dw_v,
                     double *dgamma_h, double *dgamma_k, double *dconv_w);
void orc_table_grad(const uint32_t *idx, int64_t n_tok, int32_t n_tables, int32_t head_dim, const double *demb,
                    uint32_t *rows, double *grads, int64_t *counts);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return rng;
}
static float next_f(float scale) { return scale * ((float)(next_u64() >> 40) / (float)(1 << 24) - 0.5f); }

/* a dense operand in the requested storage: fp32 values or bf16 bit patterns */
static void *dense(int64_t n, int32_t dtype, float scale) {
    if (dtype == 1) {
        uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n);
        for (int64_t i = 0; i < n; ++i) p[i] = orc_bf16_rne(next_f(scale));
        return p;
    }
    float *p = (float *)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = next_f(scale);
    return p;
}
static float *floats(int64_t n, float base, float scale) {
    float *p = (float *)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = base + next_f(scale);
    return p;
}

static int fails = 0;
#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++fails;                                                  \
        }                                                             \
    } while (0)

static void layer_case(int64_t batch, int64_t seqlen, int32_t d, int32_t heads, int32_t head_dim, int32_t n_br,
                       int32_t conv_k, int32_t conv_mode, int32_t dtype, int with_state) {
    const int32_t vocab = 97, vocab_comp = 75, n_orders = 2, orders[2] = {2, 3};
    const int32_t n_tables = n_orders * heads, De = n_tables * head_dim;
    const int64_t n_tok = batch * seqlen;
    uint32_t *primes = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n_tables);
    for (int32_t t = 0; t < n_tables; ++t) primes[t] = (uint32_t[]){101, 89, 67, 53, 41, 29, 17, 13}[t % 8];
    int32_t *comp = (int32_t *)malloc(sizeof(int32_t) * vocab);
    for (int32_t i = 0; i < vocab; ++i) comp[i] = i % vocab_comp;
    int32_t *tokens = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_tok);
    for (int64_t i = 0; i < n_tok; ++i) tokens[i] = (int32_t)(next_u64() % (vocab + 3)) - 1; /* some out of range */
    int32_t *ctx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(batch * 2));
    for (int64_t i = 0; i < batch * 2; ++i) ctx[i] = (int32_t)(next_u64() % (vocab_comp + 1));
    uint32_t *idx = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(n_tok * n_tables));
    int32_t *new_ctx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(batch * 2));
    int64_t bad = orc_hash(tokens, batch, seqlen, comp, vocab, vocab_comp, with_state ? ctx : NULL, n_orders, orders,
                           heads, primes, 0x454E4752414D0001ull, idx, new_ctx);
    CHECK(bad >= 0 && bad <= n_tok);
    for (int64_t i = 0; i < n_tok * n_tables; ++i) CHECK(idx[i] < primes[i % n_tables]);

    const size_t es = dtype == 1 ? 2 : 4;
    void *emb = malloc(es * (size_t)(n_tok * De));
    orc_gather_synth(idx, n_tok, n_tables, head_dim, 3, dtype, emb);
    /* the same rows from host tables of exactly primes[tau] rows */
    void **tabs = (void **)malloc(sizeof(void *) * (size_t)n_tables);
    for (int32_t t = 0; t < n_tables; ++t) tabs[t] = dense((int64_t)primes[t] * head_dim, dtype, 0.04f);
    void *emb2 = malloc(es * (size_t)(n_tok * De));
    orc_gather_host(idx, n_tok, n_tables, head_dim, (const void *const *)tabs, dtype, emb2);

    void *h = dense((int64_t)n_br * n_tok * d, dtype, 2.f);
    void *w_k = dense((int64_t)n_br * d * De, dtype, 0.5f);
    void *w_v = dense((int64_t)d * De, dtype, 20.f);
    float *gh = floats((int64_t)n_br * d, 1.f, 0.2f), *gk = floats((int64_t)n_br * d, 1.f, 0.2f);
    float *cw = floats((int64_t)d * conv_k, 0.f, 1.f);
    float *state = with_state && conv_k > 1 ? floats((int64_t)n_br * batch * (conv_k - 1) * d, 0.f, 1.f) : NULL;

    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    orc_project(emb, w_v, d, De, dtype, y);
    double *u1 = (double *)malloc(sizeof(double) * (size_t)d);
    double a = orc_gate_token(emb, h, w_k, w_v, gh, gk, d, De, 1e-6, dtype, u1);
    CHECK(a > 0.0 && a <= 1.0);

    /* every position of every sequence, whole and in two pieces */
    double *out = (double *)malloc(sizeof(double) * (size_t)(n_br * seqlen * d));
    double *alpha = (double *)malloc(sizeof(double) * (size_t)(n_br * seqlen));
    double *u = (double *)malloc(sizeof(double) * (size_t)(n_br * seqlen * d));
    for (int64_t b = 0; b < batch; ++b) {
        CHECK(orc_forward_range(b, 0, seqlen, batch, seqlen, d, De, n_br, conv_k, conv_mode, 1e-6, 0, dtype, emb, h,
                                w_k, w_v, gh, gk, cw, state, out, alpha, u) == 0);
        if (seqlen > 1)
            CHECK(orc_forward_range(b, seqlen / 2, seqlen, batch, seqlen, d, De, n_br, conv_k, conv_mode, 1e-6, 1,
                                    dtype, emb, h, w_k, w_v, gh, gk, cw, state, out, NULL, NULL) == 0);
    }
    CHECK(orc_forward_range(batch, 0, 1, batch, seqlen, d, De, n_br, conv_k, conv_mode, 1e-6, 0, dtype, emb, h, w_k,
                            w_v, gh, gk, cw, state, out, alpha, u) != 0); /* b out of range: rejected */
    if (conv_k > 1) {
        const int64_t tail = seqlen < conv_k - 1 ? seqlen : conv_k - 1;
        double *ut = (double *)malloc(sizeof(double) * (size_t)(n_br * batch * tail * d));
        for (int64_t i = 0; i < n_br * batch * tail * d; ++i) ut[i] = next_f(1.f);
        float *st_out = (float *)malloc(sizeof(float) * (size_t)(n_br * batch * (conv_k - 1) * d));
        orc_conv_state_update(batch, seqlen, d, n_br, conv_k, ut, state, st_out);
        free(ut);
        free(st_out);
    }

    void *dout = dense((int64_t)n_br * n_tok * d, dtype, 1.f);
    double *dh = (double *)malloc(sizeof(double) * (size_t)(n_br * n_tok * d));
    double *demb = (double *)malloc(sizeof(double) * (size_t)(n_tok * De));
    double *dwk = (double *)malloc(sizeof(double) * (size_t)((int64_t)n_br * d * De));
    double *dwv = (double *)malloc(sizeof(double) * (size_t)((int64_t)d * De));
    double *dgh = (double *)malloc(sizeof(double) * (size_t)(n_br * d));
    double *dgk = (double *)malloc(sizeof(double) * (size_t)(n_br * d));
    double *dcw = (double *)malloc(sizeof(double) * (size_t)(d * conv_k));
    CHECK(orc_backward(batch, seqlen, d, De, n_br, conv_k, conv_mode, 1e-6, 0, dtype, emb, h, w_k, w_v, gh, gk, cw,
                       dout, dh, demb, dwk, dwv, dgh, dgk, dcw) == 0);
    uint32_t *rows = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(n_tables * n_tok));
    double *grads = (double *)malloc(sizeof(double) * (size_t)(n_tables * n_tok * head_dim));
    int64_t *counts = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_tables);
    orc_table_grad(idx, n_tok, n_tables, head_dim, demb, rows, grads, counts);
    for (int32_t t = 0; t < n_tables; ++t) CHECK(counts[t] >= 1 && counts[t] <= n_tok);

    free(rows); free(grads); free(counts);
    free(dout); free(dh); free(demb); free(dwk); free(dwv); free(dgh); free(dgk); free(dcw);
    free(out); free(alpha); free(u); free(y); free(u1);
    free(h); free(w_k); free(w_v); free(gh); free(gk); free(cw); free(state);
    for (int32_t t = 0; t < n_tables; ++t) free(tabs[t]);
    free(tabs); free(emb); free(emb2);
    free(primes); free(comp); free(tokens); free(ctx); free(idx); free(new_ctx);
}

int main(void) {
    uint64_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, blk[4];
    orc_philox4x64_10(ctr, key, blk);
    CHECK(orc_mix64(0x9E3779B97F4A7C15ull) == 0xE220A8397B1DCDAFull);
    CHECK(orc_table_seed(0, 0) == 0xE220A8397B1DCDAFull);
    int32_t g[3] = {1, 2, 3};
    CHECK(orc_ngram_key(g, 3, 5) == (uint64_t)(1 * 36 + 2 * 6 + 3));
    CHECK(orc_ngram_slot(g, 3, 5, 7, 13) < 13);
    CHECK(orc_synth_value(3, 1, 77, 5) == orc_synth_value(3, 1, 77, 5));

    /* batch, seqlen, d, heads, head_dim, branches, conv_k, mode, dtype, state */
    layer_case(2, 9, 24, 2, 8, 2, 4, 0, 0, 1);
    layer_case(3, 1, 16, 1, 8, 1, 4, 1, 1, 1);
    layer_case(1, 2, 16, 4, 4, 3, 3, 0, 1, 1);
    layer_case(2, 7, 8, 2, 4, 1, 1, 1, 0, 0);
    layer_case(2, 5, 12, 3, 4, 4, 2, 0, 1, 0);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
