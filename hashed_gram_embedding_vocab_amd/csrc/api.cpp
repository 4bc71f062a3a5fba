// api.cpp -- host side of the C ABI declared in include/engram.h: plans,
// retrieval and fusion (argument validation, workspace layout and launch
// sequencing on the caller's stream), profiling and synthetic tables.  No
// entry point here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "engram.h"
#include "engram_synth.h"
#include "host_internal.h"

using namespace engram;
using namespace engram::host;

namespace {

// SplitMix64 output function, used to derive the per-table hash seeds.
struct Layout {
    size_t idx, emb, partials, alpha, v, seam, kbuf, stage, total;
};

int32_t n_parts_of(const engram_plan_s &p) {
    return p.cfg.dtype == ENGRAM_BF16 ? p.cfg.d_model / kPartCols : 1;
}

// Whether the W_v projection carries the rest of the fusion step in its
// epilogue (v never stored).  Its epilogue addresses h and out of all
// branches through one buffer resource each, with rows it must not write
// sent 2^31 bytes past the start (so h and out of all branches stay below
// 2^31 bytes), and the conv state through 32-bit offsets; it writes only the
// state rows of its own positions, so a chunk shorter than K_c - 1 (which
// also keeps rows of the old state) takes the fusion kernel.
bool fused_value_path(const engram_plan_s &p, int64_t batch, int64_t seqlen) {
    const int64_t Br = p.cfg.n_branches, d = p.cfg.d_model, kc = p.cfg.conv_kernel;
    return p.cfg.dtype == ENGRAM_BF16 && seqlen >= kc - 1 &&
           Br * batch * seqlen * d * 2 < ((int64_t)1 << 31) &&
           Br * batch * (kc - 1) * d * 4 < ((int64_t)1 << 32);
}

bool layout_of(const engram_plan_s &p, int64_t batch, int64_t seqlen, Layout &L) {
    if (batch <= 0 || seqlen <= 0) return false;
    const int64_t n_tok = batch * seqlen;
    const int64_t d = p.cfg.d_model, Br = p.cfg.n_branches;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    L.idx = take((size_t)n_tok * p.n_tables * 4);
    L.emb = take((size_t)n_tok * p.emb_dim * p.elem);
    const bool fused_v = fused_value_path(p, batch, seqlen);
    L.partials = take((size_t)Br * n_parts_of(p) * 3 * n_tok * 4);
    L.alpha = fused_v ? take((size_t)Br * n_tok * 4) : off;
    L.v = fused_v ? off : take((size_t)n_tok * d * 4);
    L.seam = fused_v ? take((size_t)((n_tok + kTokTile - 1) / kTokTile) * 6 * d * 4) : off;
    L.kbuf = p.cfg.dtype == ENGRAM_F32 ? take((size_t)Br * n_tok * d * 4) : off;
    L.stage = take((size_t)Br * batch * (p.cfg.conv_kernel - 1) * d * 4);
    L.total = off;
    return true;
}

engram_status check_hash_args(const engram_plan_s *p, const int32_t *tokens, int32_t batch,
                              int32_t seqlen, const int32_t *comp_map, uint32_t *idx) {
    if (!p || !tokens || !comp_map || !idx) return ENGRAM_E_INVALID_ARG;
    if (batch <= 0 || seqlen <= 0) return ENGRAM_E_INVALID_ARG;
    if ((int64_t)batch * seqlen > (int64_t)INT32_MAX) return ENGRAM_E_UNSUPPORTED;
    if (!aligned16(tokens) || !aligned16(comp_map) || !aligned16(idx)) return ENGRAM_E_INVALID_ARG;
    return ENGRAM_OK;
}

engram_status do_hash(engram_plan_s &p, const int32_t *tokens, int32_t batch, int32_t seqlen,
                      const int32_t *comp_map, const int32_t *prev_ctx, uint32_t *idx, uint32_t *bad,
                      hipStream_t s) {
    {
        Launch l(p, ENGRAM_K_HASH, s);
        launch_hash(p.hc, tokens, batch, seqlen, comp_map, prev_ctx, idx, bad, s);
    }
    return last_launch_status();
}


engram_status do_hash_gather(engram_plan_s &p, const int32_t *tokens, int32_t batch, int32_t seqlen,
                             const int32_t *comp_map, const int32_t *prev_ctx, uint32_t *bad,
                             const void *const *tables, void *emb, hipStream_t s, int32_t *ctx_out = nullptr) {
    const GatherConsts gc = gather_consts(p, tables);
    {
        Launch l(p, ENGRAM_K_GATHER, s);
        launch_hash_gather(p.hc, gc, tokens, batch, seqlen, comp_map, prev_ctx, bad, emb, s, ctx_out);
    }
    return last_launch_status();
}

engram_status check_fuse_args(const engram_plan_s *p, const void *emb, const void *h, int32_t batch,
                              int32_t seqlen, const engram_weights *w, const void *out,
                              const float *alpha, const void *conv_state, uint32_t flags,
                              const void *ws, size_t ws_bytes) {
    if (!p || !emb || !h || !w || !out || !ws) return ENGRAM_E_INVALID_ARG;
    if (batch <= 0 || seqlen <= 0) return ENGRAM_E_INVALID_ARG;
    if ((int64_t)batch * seqlen > (int64_t)INT32_MAX) return ENGRAM_E_UNSUPPORTED;
    if (batch > 65535) return ENGRAM_E_UNSUPPORTED;  // one grid row per sequence in the fusion kernel
    if (flags & ~(uint32_t)(ENGRAM_OUT_DELTA | ENGRAM_WEIGHTS_PACKED)) return ENGRAM_E_INVALID_ARG;
    // packed weights are read by the bf16 MFMA projections only
    if ((flags & ENGRAM_WEIGHTS_PACKED) && p->cfg.dtype != ENGRAM_BF16) return ENGRAM_E_UNSUPPORTED;
    if (!aligned16(emb) || !aligned16(h) || !aligned16(out)) return ENGRAM_E_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return ENGRAM_E_INVALID_ARG;
    if ((alpha && !aligned16(alpha)) || (conv_state && !aligned16(conv_state))) return ENGRAM_E_INVALID_ARG;
    for (int m = 0; m < p->cfg.n_branches; ++m) {
        if (!w->w_k[m] || !w->gamma_h[m] || !w->gamma_k[m]) return ENGRAM_E_INVALID_ARG;
        if (!aligned16(w->w_k[m]) || !aligned16(w->gamma_h[m]) || !aligned16(w->gamma_k[m]))
            return ENGRAM_E_INVALID_ARG;
    }
    if (!w->w_v || !w->conv_w || !aligned16(w->w_v)) return ENGRAM_E_INVALID_ARG;
    Layout L;
    if (!layout_of(*p, batch, seqlen, L) || ws_bytes < L.total) return ENGRAM_E_INVALID_ARG;
    // bf16 MFMA tiles: 256 weight rows never straddle two matrices, and the
    // K loop runs an even number of 64-wide stages
    if (p->cfg.dtype == ENGRAM_BF16 && (p->cfg.d_model % 256 != 0 || p->emb_dim % 128 != 0))
        return ENGRAM_E_UNSUPPORTED;
    // the projection kernel addresses E, each weight matrix and each
    // branch of h with 32-bit offsets
    if ((int64_t)batch * seqlen * p->emb_dim * p->elem >= ((int64_t)1 << 31) ||
        (int64_t)p->cfg.d_model * p->emb_dim * p->elem >= ((int64_t)1 << 31) ||
        (p->cfg.dtype == ENGRAM_BF16 && (int64_t)batch * seqlen * p->cfg.d_model * 2 >= ((int64_t)1 << 32)))
        return ENGRAM_E_UNSUPPORTED;
    return ENGRAM_OK;
}

// Retrieval done by the projection launch itself (short chunks): what it needs.
struct InLaunchRetrieval {
    const int32_t *tokens;
    const int32_t *comp_map;
    const int32_t *prev_ctx;
    uint32_t *bad;
    const void *const *tables;
};

// Whether engram_forward leaves retrieval to the projection launch: the
// fusion-kernel route (W_k and W_v in one launch) on 128 x 128 tiles, where
// a separate retrieval kernel would be a latency-bound launch of its own.
bool retrieval_in_projection(const engram_plan_s &p, int32_t batch, int32_t seqlen) {
    if (p.cfg.dtype != ENGRAM_BF16) return false;
    ProjArgs pa{};
    pa.d = p.cfg.d_model;
    pa.n_tok = (int64_t)batch * seqlen;
    pa.K = p.emb_dim;
    if (fused_value_path(p, batch, seqlen)) {
        // the W_k launch and the fused W_v launch both retrieve
        pa.n_mats = p.cfg.n_branches;
        return proj_gather_tables_ok(pa, p.n_tables);
    }
    pa.n_mats = p.cfg.n_branches + 1;
    return proj_gather_ok(pa, p.n_tables);
}

engram_status do_fuse(engram_plan_s &p, const void *emb, const void *h, int32_t batch, int32_t seqlen,
                      const engram_weights *w, void *conv_state, void *out, float *alpha,
                      uint32_t flags, void *ws, hipStream_t s,
                      const CtxUpdate &ctx = CtxUpdate{}, const InLaunchRetrieval *rin = nullptr) {
    Layout L;
    layout_of(p, batch, seqlen, L);
    char *base = static_cast<char *>(ws);
    const int64_t n_tok = (int64_t)batch * seqlen;
    const int Br = p.cfg.n_branches;

    ProjArgs pa{};
    pa.emb = emb;
    pa.w_packed = (flags & ENGRAM_WEIGHTS_PACKED) ? 1 : 0;
    for (int m = 0; m < Br; ++m) {
        pa.w[m] = w->w_k[m];
        pa.gamma_h[m] = w->gamma_h[m];
        pa.gamma_k[m] = w->gamma_k[m];
    }
    for (int m = Br; m < kMaxBranches; ++m) {  // unused slots: any valid pointer
        pa.gamma_h[m] = w->gamma_h[0];
        pa.gamma_k[m] = w->gamma_k[0];
    }
    pa.w[Br] = w->w_v;
    for (int m = Br + 1; m <= kMaxBranches; ++m) pa.w[m] = w->w_v;
    pa.h = h;
    pa.partials = reinterpret_cast<float *>(base + L.partials);
    pa.v = reinterpret_cast<float *>(base + L.v);
    pa.kbuf = p.cfg.dtype == ENGRAM_F32 ? reinterpret_cast<float *>(base + L.kbuf) : nullptr;
    pa.n_tok = n_tok;
    pa.K = p.emb_dim;
    pa.d = p.cfg.d_model;
    pa.n_branches = Br;
    pa.n_parts = n_parts_of(p);
    float *stage = (conv_state && p.cfg.conv_kernel > 1) ? reinterpret_cast<float *>(base + L.stage) : nullptr;
    // the gate goes straight into the caller's alpha when one is given
    float *gate = alpha ? alpha : reinterpret_cast<float *>(base + L.alpha);
    const bool fused_v = fused_value_path(p, batch, seqlen);

    // W_k of every branch (gate partials); on the fusion-kernel path W_v too
    pa.n_mats = fused_v ? Br : Br + 1;
    if (rin) {
        pa.tokens = rin->tokens;
        pa.comp_map = rin->comp_map;
        pa.prev_ctx = rin->prev_ctx;
        pa.bad = rin->bad;
        pa.seqlen = seqlen;
        pa.hc = p.hc;
        for (int t = 0; t < kMaxTables; ++t)
            pa.tables[t] = static_cast<const char *>(rin->tables[t < p.n_tables ? t : 0]);
    }
    {
        Launch l(p, ENGRAM_K_GEMM, s);
        if (rin && fused_v)
            launch_proj_k_gather_bf16(pa, s);
        else if (rin)
            launch_proj_gather_bf16(pa, s);
        else if (p.cfg.dtype == ENGRAM_BF16)
            launch_proj_bf16(pa, s);
        else
            launch_proj_f32(pa, s);
    }
    if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;

    if (fused_v) {
        // the gate of every token, which the W_v launch's epilogue reads
        // (plus the carried context, if any)
        GateArgs ga{};
        ga.partials = pa.partials;
        ga.alpha = gate;
        ga.n_tok = n_tok;
        ga.d = p.cfg.d_model;
        ga.n_branches = Br;
        ga.n_parts = pa.n_parts;
        ga.eps = p.cfg.rms_eps;
        // (with retrieval inside the launches the W_v launch still reads the
        // old context: it is rolled at the end instead)
        ga.ctx = rin ? CtxUpdate{} : ctx;
        ga.batch = batch;
        ga.seqlen = seqlen;
        {
            Launch l(p, ENGRAM_K_GATE, s);
            launch_gate(ga, s);
        }
        if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;

        // W_v with gated value, conv, residual and state in its epilogue
        ProjArgs pv = pa;
        pv.w[0] = w->w_v;
        pv.n_mats = 1;
        pv.out = out;
        pv.conv_w = w->conv_w;
        pv.conv_state = conv_state;
        pv.state_stage = stage;
        pv.state_bf16 = p.state_bf16;
        pv.alpha = gate;
        pv.seam_v = reinterpret_cast<float *>(base + L.seam);
        pv.batch = batch;
        pv.seqlen = seqlen;
        pv.conv_k = p.cfg.conv_kernel;
        pv.conv_mode = p.cfg.conv_mode;
        pv.flags = flags;
        pv.bad = nullptr;  // out-of-range ids were counted by the W_k launch
        {
            Launch l(p, ENGRAM_K_GEMM_V, s);
            if (rin)
                launch_proj_v_fused_gather_bf16(pv, s);
            else
                launch_proj_v_fused_bf16(pv, s);
        }
        const int32_t n_tiles = (int32_t)((n_tok + kTokTile - 1) / kTokTile);
        if (n_tiles > 1) {
            if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;
            SeamArgs sa{};
            sa.seam_v = pv.seam_v;
            sa.alpha = gate;
            sa.h = h;
            sa.out = out;
            sa.conv_w = w->conv_w;
            sa.conv_state = conv_state;
            sa.state_bf16 = p.state_bf16;
            sa.n_tok = n_tok;
            sa.n_tiles = n_tiles;
            sa.batch = batch;
            sa.seqlen = seqlen;
            sa.d = p.cfg.d_model;
            sa.n_branches = Br;
            sa.conv_k = p.cfg.conv_kernel;
            sa.conv_mode = p.cfg.conv_mode;
            sa.flags = flags;
            Launch l(p, ENGRAM_K_SEAM, s);
            launch_seam(sa, s);
        }
        if (rin && ctx.prev_ctx) {
            if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;
            Launch l(p, ENGRAM_K_AUX, s);
            launch_ctx_update(ctx, batch, seqlen, s);
        }
    } else {
        // a chunk of at most kFusePositions positions is one fusion-kernel
        // workgroup per sequence and channel stripe, which reads a state row
        // before it writes it: the state is updated in place
        const bool in_place = stage && seqlen <= kFusePositions;
        // the fusion kernel computes the gate itself (the same function as
        // the gate kernel), and the carried context
        FuseArgs fa{};
        fa.v = pa.v;
        fa.partials = pa.partials;
        fa.n_parts = pa.n_parts;
        fa.eps = p.cfg.rms_eps;
        fa.alpha = alpha;
        fa.ctx = ctx;
        fa.h = h;
        fa.out = out;
        fa.conv_w = w->conv_w;
        fa.conv_state = conv_state;
        fa.state_stage = in_place ? conv_state : stage;
        fa.state_bf16 = p.state_bf16;
        fa.stage_bf16 = in_place && p.state_bf16;
        if (in_place) stage = nullptr;
        fa.batch = batch;
        fa.seqlen = seqlen;
        fa.d = p.cfg.d_model;
        fa.n_branches = Br;
        fa.conv_k = p.cfg.conv_kernel;
        fa.conv_mode = p.cfg.conv_mode;
        fa.flags = flags;
        Launch l(p, ENGRAM_K_FUSE, s);
        launch_fuse(fa, p.cfg.dtype, s);
    }
    if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;
    if (stage) {
        // the staged rows (fp32) become the new state
        Launch l(p, ENGRAM_K_AUX, s);
        const int64_t n = (int64_t)Br * batch * (p.cfg.conv_kernel - 1) * p.cfg.d_model;
        if (p.state_bf16)
            launch_f32_to_bf16(stage, static_cast<uint16_t *>(conv_state), n, s);
        else
            launch_copy_f32(stage, static_cast<float *>(conv_state), n, s);
    }
    return ENGRAM_OK;
}

}  // namespace

namespace engram {
namespace host {

engram_status check_gather_args(const engram_plan_s *p, const uint32_t *idx, int64_t n_tok,
                                const void *const *tables, const void *emb) {
    if (!p || !idx || !tables || !emb) return ENGRAM_E_INVALID_ARG;
    if (n_tok <= 0) return ENGRAM_E_INVALID_ARG;
    if (!aligned16(idx) || !aligned16(emb)) return ENGRAM_E_INVALID_ARG;
    const int64_t chunks = (int64_t)p->emb_dim * p->elem / 16;
    if (n_tok > ((int64_t)1 << 40) / chunks) return ENGRAM_E_UNSUPPORTED;
    for (int t = 0; t < p->n_tables; ++t)
        if (!tables[t] || !aligned16(tables[t])) return ENGRAM_E_INVALID_ARG;
    return ENGRAM_OK;
}

GatherConsts gather_consts(const engram_plan_s &p, const void *const *tables) {
    GatherConsts gc{};
    gc.n_tables = p.n_tables;
    gc.row_chunks = p.cfg.head_dim * p.elem / 16;
    gc.tok_chunks = gc.row_chunks * p.n_tables;
    for (int t = 0; t < p.n_tables; ++t) {
        gc.table[t] = static_cast<const char *>(tables[t]);
        gc.last_row[t] = p.cfg.table_rows[t] - 1;
    }
    auto magic = [](int32_t dv) -> uint64_t {
        return dv <= 1 ? 0 : (uint64_t)(((unsigned __int128)1 << 64) / (unsigned)dv) + 1;
    };
    gc.magic_tok = magic(gc.tok_chunks);
    gc.magic_row = magic(gc.row_chunks);
    return gc;
}

engram_status do_gather(engram_plan_s &p, const uint32_t *idx, int64_t n_tok,
                        const void *const *tables, void *emb, hipStream_t s) {
    const GatherConsts gc = gather_consts(p, tables);
    {
        Launch l(p, ENGRAM_K_GATHER, s);
        launch_gather(gc, idx, n_tok, emb, s);
    }
    return last_launch_status();
}

}  // namespace host
}  // namespace engram

LaunchEvents &engram::launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}

extern "C" {

const char *engram_status_string(engram_status s) {
    switch (s) {
        case ENGRAM_OK: return "ok";
        case ENGRAM_E_INVALID_ARG: return "invalid argument";
        case ENGRAM_E_UNSUPPORTED: return "unsupported shape";
        case ENGRAM_E_DEVICE: return "device error";
        case ENGRAM_E_NOMEM: return "out of host memory";
    }
    return "unknown status";
}

engram_status engram_plan_create(const engram_config *cfg, engram_plan *out) {
    if (!cfg || !out) return ENGRAM_E_INVALID_ARG;
    *out = nullptr;
    const engram_config &c = *cfg;
    if (c.vocab <= 0 || c.vocab_comp <= 0 || c.vocab_comp >= (1 << 21)) return ENGRAM_E_INVALID_ARG;
    if (c.n_orders < 1 || c.n_orders > 2 || c.heads < 1) return ENGRAM_E_INVALID_ARG;
    for (int o = 0; o < c.n_orders; ++o)
        if (c.orders[o] != 2 && c.orders[o] != 3) return ENGRAM_E_INVALID_ARG;
    if (c.n_orders == 2 && c.orders[0] == c.orders[1]) return ENGRAM_E_INVALID_ARG;
    const int n_tables = c.n_orders * c.heads;
    if (n_tables > ENGRAM_MAX_TABLES) return ENGRAM_E_INVALID_ARG;
    if (c.dtype != ENGRAM_F32 && c.dtype != ENGRAM_BF16) return ENGRAM_E_INVALID_ARG;
    const int elem = c.dtype == ENGRAM_BF16 ? 2 : 4;
    if (c.head_dim <= 0 || (c.head_dim * elem) % 16 != 0 || c.head_dim % 4 != 0) return ENGRAM_E_INVALID_ARG;
    for (int t = 0; t < n_tables; ++t)
        if (c.table_rows[t] < 1 || c.table_rows[t] >= 0x80000000u) return ENGRAM_E_INVALID_ARG;
    if (c.d_model <= 0 || c.d_model % 8 != 0) return ENGRAM_E_INVALID_ARG;
    if (c.n_branches < 1 || c.n_branches > ENGRAM_MAX_BRANCHES) return ENGRAM_E_INVALID_ARG;
    if (c.conv_kernel < 1 || c.conv_kernel > 4) return ENGRAM_E_INVALID_ARG;
    if (c.conv_mode != ENGRAM_CONV_LINEAR && c.conv_mode != ENGRAM_CONV_SILU_SKIP) return ENGRAM_E_INVALID_ARG;
    if (!(c.rms_eps >= 0.f)) return ENGRAM_E_INVALID_ARG;
    if (c.state_dtype != ENGRAM_F32 && !(c.state_dtype == ENGRAM_BF16 && c.dtype == ENGRAM_BF16))
        return ENGRAM_E_INVALID_ARG;

    engram_plan_s *p = new (std::nothrow) engram_plan_s();
    if (!p) return ENGRAM_E_NOMEM;
    p->cfg = c;
    p->n_tables = n_tables;
    p->emb_dim = n_tables * c.head_dim;
    p->elem = elem;
    p->state_bf16 = c.state_dtype == ENGRAM_BF16;
    p->hc.n_tables = n_tables;
    p->hc.vocab = c.vocab;
    p->hc.vocab_comp = c.vocab_comp;
    for (int t = 0; t < n_tables; ++t) {
        p->hc.seed[t] = engram::table_seed(c.hash_seed, t);
        p->hc.rows[t] = c.table_rows[t];
        p->hc.magic[t] = engram::mod_magic(c.table_rows[t]);
        p->hc.order_of[t] = c.orders[t / c.heads];
    }
    *out = p;
    return ENGRAM_OK;
}

engram_status engram_plan_destroy(engram_plan p) {
    if (!p) return ENGRAM_E_INVALID_ARG;
    for (hipEvent_t e : p->prof_ev) (void)hipEventDestroy(e);
    delete p;
    return ENGRAM_OK;
}

size_t engram_workspace_size(engram_plan p, int32_t batch, int32_t seqlen) {
    Layout L;
    if (!p || !layout_of(*p, batch, seqlen, L)) return 0;
    return L.total;
}

engram_status engram_pack_weight(engram_plan p, const void *d_w, void *d_packed, hipStream_t stream) {
    if (!p || !d_w || !d_packed || !aligned16(d_w) || !aligned16(d_packed)) return ENGRAM_E_INVALID_ARG;
    if (p->cfg.dtype != ENGRAM_BF16) return ENGRAM_E_UNSUPPORTED;
    const int64_t rows = p->cfg.d_model, K = p->emb_dim;
    // the shapes the bf16 projections take (engram_gate_fuse rejects the rest)
    if (rows % 256 != 0 || K % 128 != 0 || rows * K * 2 >= ((int64_t)1 << 31)) return ENGRAM_E_UNSUPPORTED;
    const uintptr_t a = reinterpret_cast<uintptr_t>(d_w), b = reinterpret_cast<uintptr_t>(d_packed);
    const uintptr_t bytes = (uintptr_t)(rows * K * 2);
    if (a < b + bytes && b < a + bytes) return ENGRAM_E_INVALID_ARG;  // overlapping buffers
    {
        Launch l(*p, ENGRAM_K_AUX, stream);
        launch_pack_weight(d_w, d_packed, (int32_t)rows, (int32_t)K, stream);
    }
    return last_launch_status();
}

engram_status engram_hash(engram_plan p, const int32_t *d_tokens, int32_t batch, int32_t seqlen,
                          const int32_t *d_comp_map, const int32_t *d_prev_ctx, uint32_t *d_idx,
                          uint32_t *d_bad_tokens, hipStream_t stream) {
    engram_status st = check_hash_args(p, d_tokens, batch, seqlen, d_comp_map, d_idx);
    if (st != ENGRAM_OK) return st;
    return do_hash(*p, d_tokens, batch, seqlen, d_comp_map, d_prev_ctx, d_idx, d_bad_tokens, stream);
}

engram_status engram_gather(engram_plan p, const uint32_t *d_idx, int64_t n_tokens,
                            const void *const *table_ptrs, void *d_emb, hipStream_t stream) {
    engram_status st = check_gather_args(p, d_idx, n_tokens, table_ptrs, d_emb);
    if (st != ENGRAM_OK) return st;
    return do_gather(*p, d_idx, n_tokens, table_ptrs, d_emb, stream);
}

 engram_status engram_gate_fuse(engram_plan p, const void *d_emb, const void *d_h, int32_t batch,
                               int32_t seqlen, const engram_weights *w, void *d_conv_state,
                               void *d_out, float *d_alpha, uint32_t flags, void *d_workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    engram_status st = check_fuse_args(p, d_emb, d_h, batch, seqlen, w, d_out, d_alpha, d_conv_state,
                                       flags, d_workspace, workspace_bytes);
    if (st != ENGRAM_OK) return st;
    return do_fuse(*p, d_emb, d_h, batch, seqlen, w, d_conv_state, d_out, d_alpha, flags, d_workspace,
                   stream);
}

engram_status engram_forward(engram_plan p, const int32_t *d_tokens, int32_t batch, int32_t seqlen,
                             const int32_t *d_comp_map, int32_t *d_prev_ctx,
                             const void *const *table_ptrs, const void *d_h,
                             const engram_weights *w, void *d_conv_state, void *d_out,
                             float *d_alpha, uint32_t flags, void *d_workspace,
                             size_t workspace_bytes, uint32_t *d_bad_tokens, hipStream_t stream) {
    if (!p || !d_workspace) return ENGRAM_E_INVALID_ARG;
    const bool in_proj = (flags & ENGRAM_RETRIEVE_IN_PROJECTION) != 0;
    flags &= ~(uint32_t)ENGRAM_RETRIEVE_IN_PROJECTION;
    Layout L;
    if (!layout_of(*p, batch, seqlen, L)) return ENGRAM_E_INVALID_ARG;
    char *base = static_cast<char *>(d_workspace);
    uint32_t *idx = reinterpret_cast<uint32_t *>(base + L.idx);
    void *emb = base + L.emb;
    engram_status st = check_hash_args(p, d_tokens, batch, seqlen, d_comp_map, idx);
    if (st == ENGRAM_OK) st = check_gather_args(p, idx, (int64_t)batch * seqlen, table_ptrs, emb);
    if (st == ENGRAM_OK)
        st = check_fuse_args(p, emb, d_h, batch, seqlen, w, d_out, d_alpha, d_conv_state, flags,
                             d_workspace, workspace_bytes);
    if (st != ENGRAM_OK) return st;
    // the carried context is updated by a later kernel of this call, after
    // retrieval has read the old one
    CtxUpdate ctx{};
    ctx.tokens = d_tokens;
    ctx.comp_map = d_comp_map;
    ctx.prev_ctx = d_prev_ctx;
    ctx.vocab = p->cfg.vocab;
    ctx.vocab_comp = p->cfg.vocab_comp;
    if (in_proj && retrieval_in_projection(*p, batch, seqlen)) {
        // short chunks: the projection launch hashes and gathers itself
        const InLaunchRetrieval rin{d_tokens, d_comp_map, d_prev_ctx, d_bad_tokens, table_ptrs};
        return do_fuse(*p, emb, d_h, batch, seqlen, w, d_conv_state, d_out, d_alpha, flags, d_workspace, stream,
                       ctx, &rin);
    }
    // retrieval in one kernel: hash every (token, table) pair and copy its row
    st = do_hash_gather(*p, d_tokens, batch, seqlen, d_comp_map, d_prev_ctx, d_bad_tokens, table_ptrs,
                        emb, stream);
    if (st != ENGRAM_OK) return st;
    return do_fuse(*p, emb, d_h, batch, seqlen, w, d_conv_state, d_out, d_alpha, flags, d_workspace,
                   stream, ctx);
}

engram_status engram_retrieve(engram_plan p, const int32_t *d_tokens, int32_t batch, int32_t seqlen,
                              const int32_t *d_comp_map, int32_t *d_prev_ctx, const void *const *table_ptrs,
                              void *d_emb, uint32_t *d_bad_tokens, hipStream_t stream) {
    if (!p || !d_tokens || !d_comp_map || !table_ptrs || !d_emb) return ENGRAM_E_INVALID_ARG;
    if (batch <= 0 || seqlen <= 0) return ENGRAM_E_INVALID_ARG;
    if ((int64_t)batch * seqlen > (int64_t)INT32_MAX) return ENGRAM_E_UNSUPPORTED;
    if (!aligned16(d_tokens) || !aligned16(d_comp_map) || !aligned16(d_emb)) return ENGRAM_E_INVALID_ARG;
    for (int t = 0; t < p->n_tables; ++t)
        if (!table_ptrs[t] || !aligned16(table_ptrs[t])) return ENGRAM_E_INVALID_ARG;
    // one token per sequence: the retrieval launch rolls the context itself
    engram_status st = do_hash_gather(*p, d_tokens, batch, seqlen, d_comp_map, d_prev_ctx, d_bad_tokens,
                                      table_ptrs, d_emb, stream, seqlen == 1 ? d_prev_ctx : nullptr);
    if (st != ENGRAM_OK || !d_prev_ctx || seqlen == 1) return st;
    // after the retrieval has read the old context, on the same stream
    const CtxUpdate ctx{d_tokens, d_comp_map, d_prev_ctx, p->cfg.vocab, p->cfg.vocab_comp};
    {
        Launch l(*p, ENGRAM_K_AUX, stream);
        launch_ctx_update(ctx, batch, seqlen, stream);
    }
    return last_launch_status();
}

engram_status engram_profile_begin(engram_plan p, int32_t max_launches, uint32_t kind_mask) {
    if (!p || max_launches <= 0) return ENGRAM_E_INVALID_ARG;
    if (kind_mask >> ENGRAM_K_COUNT) return ENGRAM_E_INVALID_ARG;
    p->prof_mask = kind_mask ? kind_mask : (1u << ENGRAM_K_COUNT) - 1u;
    if ((int32_t)p->prof_ev.size() < 2 * max_launches) {
        for (hipEvent_t e : p->prof_ev) (void)hipEventDestroy(e);
        p->prof_ev.assign(2 * max_launches, nullptr);
        for (auto &e : p->prof_ev)
            if (hipEventCreate(&e) != hipSuccess) return ENGRAM_E_DEVICE;
    }
    p->prof_kind.assign(max_launches, 0);
    for (int64_t &c : p->prof_seen) c = 0;
    p->prof_max = max_launches;
    p->prof_used = 0;
    p->prof_dropped = 0;
    p->prof_on = true;
    return ENGRAM_OK;
}

engram_status engram_profile_every(engram_plan p, int32_t every) {
    if (!p || every < 1) return ENGRAM_E_INVALID_ARG;
    p->prof_every = every;
    return ENGRAM_OK;
}

engram_status engram_profile_end(engram_plan p, engram_profile *out) {
    if (!p || !out) return ENGRAM_E_INVALID_ARG;
    std::memset(out, 0, sizeof(*out));
    p->prof_on = false;
    engram_status st = ENGRAM_OK;
    for (int32_t i = 0; i < p->prof_used; ++i) {
        if (p->prof_kind[i] < 0) continue;
        float ms = 0.f;
        if (hipEventSynchronize(p->prof_ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, p->prof_ev[2 * i], p->prof_ev[2 * i + 1]) != hipSuccess) {
            st = ENGRAM_E_DEVICE;
            continue;
        }
        out->total_ms[p->prof_kind[i]] += ms;
        out->launches[p->prof_kind[i]] += 1;
    }
    out->dropped = p->prof_dropped;
    p->prof_used = 0;
    return st;
}

engram_status engram_synth_fill_table(int32_t dtype, uint64_t seed, int32_t tau, int64_t rows,
                                      int32_t head_dim, void *d_table, hipStream_t stream) {
    if (!d_table || rows <= 0 || head_dim <= 0 || head_dim % 4 != 0 || tau < 0) return ENGRAM_E_INVALID_ARG;
    if (dtype != ENGRAM_F32 && dtype != ENGRAM_BF16) return ENGRAM_E_INVALID_ARG;
    if (!aligned16(d_table)) return ENGRAM_E_INVALID_ARG;
    launch_synth_fill((engram_dtype)dtype, seed, tau, rows, head_dim, d_table, stream);
    return last_launch_status();
}

engram_status engram_probe_stream(int32_t mode, uint32_t flags, int32_t unroll, int32_t blocks,
                                  const void *d_src, void *d_dst, int64_t bytes, hipStream_t stream) {
    if (mode != 0 && mode != 1) return ENGRAM_E_INVALID_ARG;
    if ((flags & ~(uint32_t)ENGRAM_PROBE_NONTEMPORAL) != 0) return ENGRAM_E_INVALID_ARG;
    if (unroll != 4 && unroll != 8 && unroll != 16) return ENGRAM_E_INVALID_ARG;
    if (blocks < 1 || blocks > (1 << 20)) return ENGRAM_E_INVALID_ARG;
    if (!d_src || !d_dst || !aligned16(d_src) || !aligned16(d_dst)) return ENGRAM_E_INVALID_ARG;
    if (bytes <= 0 || bytes % 16 != 0) return ENGRAM_E_INVALID_ARG;
    if (!launch_stream_probe(mode, (flags & ENGRAM_PROBE_NONTEMPORAL) != 0, unroll, d_src, d_dst, bytes, blocks,
                             stream))
        return ENGRAM_E_INVALID_ARG;
    return last_launch_status();
}

}  // extern "C"
