// api_backward.cpp -- host side of engram_backward (include/engram.h): the
// shapes it covers, its workspace layout and the launch sequence of one
// layer's gradients on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "host_internal.h"

using namespace engram;
using namespace engram::host;

namespace {

struct BwdLayout {
    size_t E, KV, parts, stats, dalpha, dconv, dg, dkv, demb, keys_in, keys_out, vals_in, vals_out, head,
        incl, temp, sum_part, dw_part, lead, tail, cflags, tinfo, total;
    size_t temp_bytes;
    int64_t n_pad;
    int32_t n_stripes, conv_blocks, gate_chunks, dw_splits;
};

// The shapes engram_backward covers (status ENGRAM_OK), with its workspace.
engram_status bwd_layout_of(const engram_plan_s &p, int32_t batch, int32_t seqlen, BwdLayout &L) {
    if (batch <= 0 || seqlen <= 0) return ENGRAM_E_INVALID_ARG;
    if (p.cfg.dtype != ENGRAM_BF16 || p.cfg.d_model % 256 != 0 || p.emb_dim % 128 != 0 || p.cfg.head_dim > 256)
        return ENGRAM_E_UNSUPPORTED;
    const int64_t n_tok = (int64_t)batch * seqlen;
    const int64_t d = p.cfg.d_model, Br = p.cfg.n_branches, De = p.emb_dim, N = (Br + 1) * d;
    const int64_t n_pad = (n_tok + 127) / 128 * 128;
    const int64_t lim = (int64_t)1 << 31;  // the MFMA loop addresses each operand with 32-bit offsets
    if (n_tok * N * 2 >= lim || n_pad * N * 2 >= lim || n_pad * De * 2 >= lim || n_tok * De * 2 >= lim ||
        d * De * 2 >= lim || n_tok * p.n_tables >= ((int64_t)1 << 32))
        return ENGRAM_E_UNSUPPORTED;
    L.n_pad = n_pad;
    L.n_stripes = (int32_t)((d + 1023) / 1024);
    L.conv_blocks = bwd_conv_blocks(batch, seqlen);
    L.gate_chunks = bwd_gate_chunks(n_tok);
    const int64_t n_items = n_tok * p.n_tables;
    L.temp_bytes = bwd_table_temp_bytes(n_items);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    L.E = take((size_t)(n_tok * De * 2));
    L.KV = take((size_t)(n_tok * N * 4));
    L.parts = take((size_t)(Br * (d / 128) * 3 * n_tok * 4));
    L.stats = take((size_t)(4 * Br * n_tok * 4));
    L.dalpha = take((size_t)(Br * L.n_stripes * n_tok * 4));
    L.dconv = take((size_t)L.conv_blocks * (size_t)(d * p.cfg.conv_kernel * 4));
    L.dg = take((size_t)(2 * Br * L.gate_chunks * d * 4));
    L.dkv = take((size_t)(n_tok * N * 2));
    L.demb = take((size_t)(n_tok * De * 4));
    L.keys_in = take((size_t)n_items * 8);
    L.keys_out = take((size_t)n_items * 8);
    L.vals_in = take((size_t)n_items * 4);
    L.vals_out = take((size_t)n_items * 4);
    L.head = take((size_t)n_items * 4);
    L.incl = take((size_t)n_items * 4);
    L.temp = take(L.temp_bytes);
    const int64_t slabs = std::max(bwd_sum_slabs(L.gate_chunks), bwd_sum_slabs(L.conv_blocks));
    L.sum_part = take((size_t)(std::max(Br * d, d * p.cfg.conv_kernel) * slabs * 4));
    L.dw_splits = plain_k_splits(N, De, n_pad);
    L.dw_part = take(L.dw_splits > 1 ? (size_t)(L.dw_splits * N * De * 4) : 0);
    const int64_t chunks = bwd_row_chunks(n_items);
    L.lead = take((size_t)(chunks * p.cfg.head_dim * 4));
    L.tail = take((size_t)(chunks * p.cfg.head_dim * 4));
    L.cflags = take((size_t)(chunks * 4));
    L.tinfo = take((size_t)(chunks * 8));
    L.total = off;
    return ENGRAM_OK;
}

}  // namespace

extern "C" {


size_t engram_backward_workspace_size(engram_plan p, int32_t batch, int32_t seqlen) {
    BwdLayout L;
    if (!p || bwd_layout_of(*p, batch, seqlen, L) != ENGRAM_OK) return 0;
    return L.total;
}

engram_status engram_backward(engram_plan p, const uint32_t *d_idx, const void *const *table_ptrs,
                              const void *d_h, const engram_weights *w, const void *d_dout, int32_t batch,
                              int32_t seqlen, uint32_t flags, void *d_dh, const engram_grads *g, void *d_workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (!p || !d_h || !w || !d_dout || !d_dh || !g || !d_workspace) return ENGRAM_E_INVALID_ARG;
    if (flags & ~(uint32_t)ENGRAM_OUT_DELTA) return ENGRAM_E_INVALID_ARG;
    BwdLayout L;
    engram_status st = bwd_layout_of(*p, batch, seqlen, L);
    if (st != ENGRAM_OK) return st;
    if (workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(d_workspace) & 255u) != 0)
        return ENGRAM_E_INVALID_ARG;
    const int64_t n_tok = (int64_t)batch * seqlen;
    st = check_gather_args(p, d_idx, n_tok, table_ptrs, d_workspace);
    if (st != ENGRAM_OK) return st;
    const int Br = p->cfg.n_branches;
    if (!aligned16(d_h) || !aligned16(d_dout) || !aligned16(d_dh) || !w->w_v || !aligned16(w->w_v) || !w->conv_w)
        return ENGRAM_E_INVALID_ARG;
    for (int m = 0; m < Br; ++m)
        if (!w->w_k[m] || !w->gamma_h[m] || !w->gamma_k[m] || !aligned16(w->w_k[m]) || !aligned16(w->gamma_h[m]) ||
            !aligned16(w->gamma_k[m]))
            return ENGRAM_E_INVALID_ARG;
    if (!g->dw || !g->dgamma_h || !g->dgamma_k || !g->dconv_w || !g->row_ids || !g->row_grads || !g->row_counts ||
        !aligned16(g->dw) || !aligned16(g->dgamma_h) || !aligned16(g->dgamma_k))
        return ENGRAM_E_INVALID_ARG;

    char *base = static_cast<char *>(d_workspace);
    const int d = p->cfg.d_model, De = p->emb_dim, kc = p->cfg.conv_kernel;
    const int64_t N = (int64_t)(Br + 1) * d;
    void *E = base + L.E;
    float *KV = reinterpret_cast<float *>(base + L.KV);
    uint16_t *dkv = reinterpret_cast<uint16_t *>(base + L.dkv);
    float *demb = reinterpret_cast<float *>(base + L.demb);
    engram_plan_s &P = *p;

    // retrieval again: E of the chunk
    st = do_gather(P, d_idx, n_tok, table_ptrs, E, stream);
    if (st != ENGRAM_OK) return st;
    // k of every branch and v, fp32, and the gate partial sums of the W_k
    // rows (the forward's: h gamma_h gamma_k k, k^2, h^2 per 128 channels)
    float *parts = reinterpret_cast<float *>(base + L.parts);
    {
        ProjArgs pa{};
        pa.emb = E;
        for (int m = 0; m <= kMaxBranches; ++m) pa.w[m] = m < Br ? w->w_k[m] : w->w_v;
        for (int m = 0; m < kMaxBranches; ++m) {
            pa.gamma_h[m] = w->gamma_h[m < Br ? m : 0];
            pa.gamma_k[m] = w->gamma_k[m < Br ? m : 0];
        }
        pa.h = d_h;
        pa.partials = parts;
        pa.n_parts = d / 128;
        pa.n_tok = n_tok;
        pa.K = De;
        pa.d = d;
        pa.n_mats = Br + 1;
        pa.n_branches = Br;
        pa.out_f32 = KV;
        pa.out_ld = N;
        pa.n_rows = (int32_t)N;
        Launch l(P, ENGRAM_K_BWD_GEMM, stream);
        launch_proj_kv_partials_bf16(pa, stream);
    }
    if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;

    BwdArgs ba{};
    ba.h = d_h;
    ba.dout = d_dout;
    ba.dh = d_dh;
    ba.kv = KV;
    ba.kv_ld = N;
    ba.stats = reinterpret_cast<float *>(base + L.stats);
    ba.partials = parts;
    ba.n_parts = d / 128;
    ba.dalpha_part = reinterpret_cast<float *>(base + L.dalpha);
    ba.dconv_part = reinterpret_cast<float *>(base + L.dconv);
    ba.dg_part = reinterpret_cast<float *>(base + L.dg);
    ba.dkv = dkv;
    ba.dkv_ld = N;
    for (int m = 0; m < kMaxBranches; ++m) {
        ba.gamma_h[m] = w->gamma_h[m < Br ? m : 0];
        ba.gamma_k[m] = w->gamma_k[m < Br ? m : 0];
    }
    ba.conv_w = w->conv_w;
    ba.n_tok = n_tok;
    ba.batch = batch;
    ba.seqlen = seqlen;
    ba.d = d;
    ba.n_branches = Br;
    ba.conv_k = kc;
    ba.conv_mode = p->cfg.conv_mode;
    ba.n_stripes = L.n_stripes;
    ba.flags = flags;
    ba.eps = p->cfg.rms_eps;
    {
        // gate statistics, the conv / gated value and the gate / RMSNorm
        // backward and the small gradients' reductions (no operand is
        // transposed: dE reads W, and dW reads E and [dk | dv], as they are)
        Launch l(P, ENGRAM_K_BWD_FUSE, stream);
        launch_bwd_gate_stats(ba, stream);
        launch_bwd_conv(ba, stream);
        launch_bwd_gate(ba, stream);
        float *part = reinterpret_cast<float *>(base + L.sum_part);
        launch_bwd_sum_rows(ba.dg_part, Br, L.gate_chunks, d, part, g->dgamma_h, stream);
        launch_bwd_sum_rows(ba.dg_part + (int64_t)Br * L.gate_chunks * d, Br, L.gate_chunks, d, part, g->dgamma_k,
                            stream);
        launch_bwd_sum_rows(ba.dconv_part, 1, L.conv_blocks, (int64_t)d * kc, part, g->dconv_w, stream);
    }
    if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;
    {
        // dE = [dk | dv] [W_k; W_v] and dW = [dk | dv]^T E on the MFMA loop
        Launch l(P, ENGRAM_K_BWD_GEMM, stream);
        ProjArgs pe{};
        pe.emb = dkv;
        for (int m = 0; m <= kMaxBranches; ++m) pe.w[m] = m < Br ? w->w_k[m] : w->w_v;
        pe.k_mat_rows = d;  // k = row of [W_k^(0); ..; W_v], d rows per matrix
        pe.w_ld = De;
        pe.n_tok = n_tok;
        pe.K = (int32_t)N;
        pe.d = De;
        pe.n_mats = 1;
        pe.out_f32 = demb;
        pe.out_ld = De;
        pe.n_rows = De;
        launch_proj_plain_kmajor_w_bf16(pe, stream);
        // dW contracts over every token: few output tiles, so K is split
        // until the chip is full and the partial results summed in order.
        // Both operands are token-major, i.e. K-major for this contraction
        // (tokens past n_tok up to n_pad read as zeros).
        ProjArgs pw{};
        pw.emb = dkv;
        for (int m = 0; m <= kMaxBranches; ++m) pw.w[m] = E;
        pw.n_tok = N;
        pw.K = (int32_t)(L.n_pad / L.dw_splits);
        pw.k_rows = n_tok;
        pw.w_ld = De;
        pw.e_ld = (int32_t)N;
        pw.d = De;
        pw.n_mats = 1;
        pw.out_f32 = L.dw_splits > 1 ? reinterpret_cast<float *>(base + L.dw_part) : g->dw;
        pw.out_ld = De;
        pw.out_split = N * De;
        pw.n_rows = De;
        launch_proj_plain_kmajor_bf16(pw, stream, L.dw_splits);
        if (L.dw_splits > 1)
            launch_bwd_sum_parts(reinterpret_cast<float *>(base + L.dw_part), 1, N * De, L.dw_splits, g->dw, stream);
    }
    if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;
    {
        BwdTableArgs ta{};
        ta.idx = d_idx;
        ta.demb = demb;
        ta.n_tok = n_tok;
        ta.n_tables = p->n_tables;
        ta.head_dim = p->cfg.head_dim;
        ta.table_rows = p->cfg.table_rows;
        ta.keys_in = base + L.keys_in;
        ta.keys_out = base + L.keys_out;
        ta.vals_in = reinterpret_cast<uint32_t *>(base + L.vals_in);
        ta.vals_out = reinterpret_cast<uint32_t *>(base + L.vals_out);
        ta.head = reinterpret_cast<uint32_t *>(base + L.head);
        ta.incl = reinterpret_cast<uint32_t *>(base + L.incl);
        ta.temp = base + L.temp;
        ta.temp_bytes = L.temp_bytes;
        ta.row_ids = g->row_ids;
        ta.row_grads = g->row_grads;
        ta.row_counts = g->row_counts;
        ta.lead = reinterpret_cast<float *>(base + L.lead);
        ta.tail = reinterpret_cast<float *>(base + L.tail);
        ta.cflags = reinterpret_cast<uint32_t *>(base + L.cflags);
        ta.tinfo = reinterpret_cast<uint32_t *>(base + L.tinfo);
        Launch l(P, ENGRAM_K_BWD_TABLE, stream);
        if (launch_bwd_table_grad(ta, stream) != hipSuccess) return ENGRAM_E_DEVICE;
    }
    return last_launch_status();
}

}  // extern "C"
