// api.cpp -- host side of the C ABI declared in include/engram.h: plans,
// argument validation, workspace layout and launch sequencing on the
// caller's stream.  No entry point allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "engram.h"
#include "engram_internal.h"
#include "engram_synth.h"

using namespace engram;

struct engram_plan_s {
    engram_config cfg;
    int32_t n_tables = 0;
    int32_t emb_dim = 0;    // D_e
    int32_t elem = 0;       // bytes per element of the plan dtype
    HashConsts hc{};
    // profiling
    bool prof_on = false;
    uint32_t prof_mask = 0;
    int32_t prof_max = 0;
    int32_t prof_used = 0;
    int64_t prof_dropped = 0;
    std::vector<hipEvent_t> prof_ev;
    std::vector<int32_t> prof_kind;
};

namespace {

// SplitMix64 output function, used to derive the per-table hash seeds.
uint64_t host_mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

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

// One timed library launch while profiling is on: hands a pair of the
// plan's events to the kernel launches in its scope (see launch_kernel).
struct Launch {
    engram_plan_s &p;
    int32_t slot = -1;
    Launch(engram_plan_s &pl, int32_t kind, hipStream_t) : p(pl) {
        if (!p.prof_on || !((p.prof_mask >> kind) & 1u)) return;
        if (p.prof_used < p.prof_max) {
            slot = p.prof_used++;
            p.prof_kind[slot] = kind;
            launch_events() = LaunchEvents{p.prof_ev[2 * slot], p.prof_ev[2 * slot + 1]};
        } else {
            ++p.prof_dropped;
        }
    }
    ~Launch() {
        if (slot < 0) return;
        if (launch_events().start != nullptr) p.prof_kind[slot] = -1;  // nothing was launched
        launch_events() = LaunchEvents{};
    }
};

engram_status last_launch_status() {
    return hipGetLastError() == hipSuccess ? ENGRAM_OK : ENGRAM_E_DEVICE;
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

engram_status do_hash_gather(engram_plan_s &p, const int32_t *tokens, int32_t batch, int32_t seqlen,
                             const int32_t *comp_map, const int32_t *prev_ctx, uint32_t *bad,
                             const void *const *tables, void *emb, hipStream_t s) {
    const GatherConsts gc = gather_consts(p, tables);
    {
        Launch l(p, ENGRAM_K_GATHER, s);
        launch_hash_gather(p.hc, gc, tokens, batch, seqlen, comp_map, prev_ctx, bad, emb, s);
    }
    return last_launch_status();
}

engram_status check_fuse_args(const engram_plan_s *p, const void *emb, const void *h, int32_t batch,
                              int32_t seqlen, const engram_weights *w, const void *out,
                              const float *alpha, const float *conv_state, uint32_t flags,
                              const void *ws, size_t ws_bytes) {
    if (!p || !emb || !h || !w || !out || !ws) return ENGRAM_E_INVALID_ARG;
    if (batch <= 0 || seqlen <= 0) return ENGRAM_E_INVALID_ARG;
    if ((int64_t)batch * seqlen > (int64_t)INT32_MAX) return ENGRAM_E_UNSUPPORTED;
    if (batch > 65535) return ENGRAM_E_UNSUPPORTED;  // one grid row per sequence in the fusion kernel
    if (flags & ~(uint32_t)ENGRAM_OUT_DELTA) return ENGRAM_E_INVALID_ARG;
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
    if (p.cfg.dtype != ENGRAM_BF16 || fused_value_path(p, batch, seqlen)) return false;
    ProjArgs pa{};
    pa.n_mats = p.cfg.n_branches + 1;
    pa.d = p.cfg.d_model;
    pa.n_tok = (int64_t)batch * seqlen;
    pa.K = p.emb_dim;
    return proj_gather_ok(pa, p.n_tables);
}

engram_status do_fuse(engram_plan_s &p, const void *emb, const void *h, int32_t batch, int32_t seqlen,
                      const engram_weights *w, float *conv_state, void *out, float *alpha,
                      uint32_t flags, void *ws, hipStream_t s,
                      const CtxUpdate &ctx = CtxUpdate{}, const InLaunchRetrieval *rin = nullptr) {
    Layout L;
    layout_of(p, batch, seqlen, L);
    char *base = static_cast<char *>(ws);
    const int64_t n_tok = (int64_t)batch * seqlen;
    const int Br = p.cfg.n_branches;

    ProjArgs pa{};
    pa.emb = emb;
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
        if (rin)
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
        ga.ctx = ctx;
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
        pv.alpha = gate;
        pv.seam_v = reinterpret_cast<float *>(base + L.seam);
        pv.batch = batch;
        pv.seqlen = seqlen;
        pv.conv_k = p.cfg.conv_kernel;
        pv.conv_mode = p.cfg.conv_mode;
        pv.flags = flags;
        {
            Launch l(p, ENGRAM_K_GEMM_V, s);
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
    } else {
        // a chunk of at most kFusePositions positions is one fusion-kernel
        // workgroup per sequence and channel stripe, which reads a state row
        // before it writes it: the state is updated in place
        if (stage && seqlen <= kFusePositions) stage = conv_state;
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
        fa.state_stage = stage;
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
    if (stage && stage != conv_state) {
        Launch l(p, ENGRAM_K_AUX, s);
        const size_t bytes = (size_t)Br * batch * (p.cfg.conv_kernel - 1) * p.cfg.d_model * 4;
        launch_copy_f32(stage, conv_state, (int64_t)(bytes / 4), s);
    }
    return ENGRAM_OK;
}

}  // namespace

LaunchEvents &engram::launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}

// ---------------------------------------------------------------- host-gather prefetcher
// The pages' deployment of host-resident tables: a step's rows are gathered
// from host DRAM by host threads and copied to the GPU by a DMA engine while
// earlier layers compute.  Until E is assembled the prefetch uses no compute
// units (a kernel queued behind a model's kernels would wait for them):
//   begin: the copy stream waits for the caller's stream, then copies the
//     indices to pinned memory.
//   worker thread and pool threads: each thread takes an equal share of the
//     (token, table) pairs, 64 at a time: the cache keys of the 64 are
//     requested, looked up (code = cache slot, or a miss), the missed rows
//     requested and copied into pinned staging, compacted from the start of
//     the thread's share.  Each thread then queues the copy of its codes and
//     staged rows to one of two device buffer sets (jobs alternate, so a job
//     never waits for the previous job's assembly) on the copy stream, so the
//     DMA of early shares overlaps the gathering of later ones.
//   finish: the caller's stream waits for those copies and assembles E.
constexpr uint32_t kPfMiss = 0x80000000u;

struct engram_prefetcher_s {
    engram_plan_s *plan = nullptr;
    GatherConsts gc{};
    const char *tables[kMaxTables] = {};
    uint32_t last_row[kMaxTables] = {};
    int32_t n_tables = 0;
    engram_row_cache cache{};
    std::vector<uint32_t> keys;   // host copy of the cache keys
    int64_t max_tok = 0;
    int32_t n_threads = 1;
    int dev = 0;
    size_t row_bytes = 0;
    // device: two buffer sets
    uint32_t *d_code[2] = {nullptr, nullptr};
    void *d_staged[2] = {nullptr, nullptr};
    // pinned host
    uint32_t *h_idx = nullptr, *h_code = nullptr;
    char *h_staged = nullptr;
    hipStream_t copy = nullptr;
    hipEvent_t ev_begin = nullptr, ev_idx = nullptr;
    hipEvent_t ev_staged[2] = {nullptr, nullptr}, ev_assembled[2] = {nullptr, nullptr};
    bool assembled[2] = {false, false};
    // job state
    std::mutex mu;
    std::condition_variable cv;
    enum State { IDLE, LISTING, STAGED } state = IDLE;
    bool stop = false;
    int64_t job_tok = 0;
    uint64_t job_count = 0;  // jobs begun; the job's buffer set is job_count & 1 at begin
    int job_set = 0;
    uint32_t job_misses = 0;
    hipError_t err = hipSuccess;
    std::thread worker;
    // host pool
    std::mutex pmu;
    std::condition_variable pcv, pdone;
    uint64_t pgen = 0;
    int pending = 0;
    int pset = 0;
    int64_t pn = 0;
    std::vector<hipError_t> terr;  // per thread
    std::vector<uint32_t> tcount;  // per thread: rows staged
    std::vector<std::thread> pool;
};

namespace {

// Cache slot of a row: the same probe sequence as the device lookups.
inline int64_t host_cache_slot(const engram_prefetcher_s *f, uint32_t tau, uint32_t row) {
    const uint32_t cap = f->cache.capacity;
    if (cap == 0) return -1;
    const uint32_t *k = f->keys.data() + (size_t)tau * cap;
    uint32_t s = (uint32_t)(((uint64_t)(row * 0x9E3779B1u) * cap) >> 32);
    for (uint32_t probe = 0; probe < cap; ++probe) {
        const uint32_t key = k[s];
        if (key == row + 1u) return (int64_t)tau * cap + s;
        if (key == 0u) return -1;
        s = s + 1u == cap ? 0u : s + 1u;
    }
    return -1;
}

// Pairs [lo, hi): codes, staged rows from position lo on, and the copies
// of both to the job's device buffers.
hipError_t pf_share(engram_prefetcher_s *f, int set, int64_t lo, int64_t hi, uint32_t &n_staged) {
    const int nt = f->n_tables;
    const size_t rb = f->row_bytes;
    const uint32_t cap = f->cache.capacity;
    constexpr int kBatch = 64;
    int64_t n = 0;  // misses staged so far
    for (int64_t b0 = lo; b0 < hi; b0 += kBatch) {
        const int cnt = (int)std::min<int64_t>(kBatch, hi - b0);
        uint32_t row[kBatch], tau[kBatch];
        for (int i = 0; i < cnt; ++i) {
            const int64_t pr = b0 + i;
            tau[i] = (uint32_t)(pr % nt);
            row[i] = std::min(f->h_idx[pr], f->last_row[tau[i]]);
            if (cap)
                __builtin_prefetch(f->keys.data() + (size_t)tau[i] * cap +
                                   (uint32_t)(((uint64_t)(row[i] * 0x9E3779B1u) * cap) >> 32));
        }
        int miss[kBatch], n_miss = 0;
        for (int i = 0; i < cnt; ++i) {
            const int64_t slot = host_cache_slot(f, tau[i], row[i]);
            if (slot >= 0) {
                f->h_code[b0 + i] = (uint32_t)slot;
            } else {
                miss[n_miss++] = i;
                __builtin_prefetch(f->tables[tau[i]] + (size_t)row[i] * rb);
            }
        }
        for (int j = 0; j < n_miss; ++j) {
            const int i = miss[j];
            const int64_t m = lo + n + j;
            std::memcpy(f->h_staged + (size_t)m * rb, f->tables[tau[i]] + (size_t)row[i] * rb, rb);
            f->h_code[b0 + i] = kPfMiss | (uint32_t)m;
        }
        n += n_miss;
    }
    n_staged = (uint32_t)n;
    hipError_t e = hipMemcpyAsync(f->d_code[set] + lo, f->h_code + lo, (size_t)(hi - lo) * 4, hipMemcpyHostToDevice,
                                  f->copy);
    if (e == hipSuccess && n > 0)
        e = hipMemcpyAsync(static_cast<char *>(f->d_staged[set]) + (size_t)lo * rb, f->h_staged + (size_t)lo * rb,
                           (size_t)n * rb, hipMemcpyHostToDevice, f->copy);
    return e;
}

void pf_range(engram_prefetcher_s *f, int t, int64_t n, int64_t &lo, int64_t &hi) {
    lo = n * t / f->n_threads;
    hi = n * (t + 1) / f->n_threads;
}

void pool_main(engram_prefetcher_s *f, int t) {
    (void)hipSetDevice(f->dev);
    uint64_t seen = 0;
    for (;;) {
        int set;
        int64_t n;
        {
            std::unique_lock<std::mutex> lk(f->pmu);
            f->pcv.wait(lk, [&] { return f->stop || f->pgen != seen; });
            if (f->stop) return;
            seen = f->pgen;
            set = f->pset;
            n = f->pn;
        }
        int64_t lo, hi;
        pf_range(f, t, n, lo, hi);
        f->terr[t] = pf_share(f, set, lo, hi, f->tcount[t]);
        {
            std::lock_guard<std::mutex> lk(f->pmu);
            if (--f->pending == 0) f->pdone.notify_all();
        }
    }
}

// Every thread's share of n pairs (this thread takes share 0); the first
// error of any thread.
hipError_t pf_run(engram_prefetcher_s *f, int set, int64_t n) {
    {
        std::lock_guard<std::mutex> lk(f->pmu);
        f->pset = set;
        f->pn = n;
        f->pending = f->n_threads - 1;
        ++f->pgen;
    }
    f->pcv.notify_all();
    int64_t lo, hi;
    pf_range(f, 0, n, lo, hi);
    f->terr[0] = pf_share(f, set, lo, hi, f->tcount[0]);
    std::unique_lock<std::mutex> lk(f->pmu);
    f->pdone.wait(lk, [&] { return f->pending == 0; });
    for (hipError_t e : f->terr)
        if (e != hipSuccess) return e;
    return hipSuccess;
}

void worker_main(engram_prefetcher_s *f) {
    (void)hipSetDevice(f->dev);
    for (;;) {
        int64_t n_tok;
        int set;
        {
            std::unique_lock<std::mutex> lk(f->mu);
            f->cv.wait(lk, [&] { return f->stop || f->state == engram_prefetcher_s::LISTING; });
            if (f->stop) return;
            n_tok = f->job_tok;
            set = f->job_set;
        }
        const int64_t n_pairs = n_tok * f->n_tables;
        hipError_t e = hipEventSynchronize(f->ev_idx);
        uint32_t n_miss = 0;
        // this set's previous assembly has read its buffers before they are refilled
        if (e == hipSuccess && f->assembled[set]) e = hipStreamWaitEvent(f->copy, f->ev_assembled[set], 0);
        if (e == hipSuccess) e = pf_run(f, set, n_pairs);
        if (e == hipSuccess) {
            e = hipEventRecord(f->ev_staged[set], f->copy);
            for (uint32_t c : f->tcount) n_miss += c;
        }
        {
            std::lock_guard<std::mutex> lk(f->mu);
            f->err = e;
            f->job_misses = n_miss;
            f->state = engram_prefetcher_s::STAGED;
        }
        f->cv.notify_all();
    }
}

void prefetcher_free(engram_prefetcher_s *f) {
    {
        std::lock_guard<std::mutex> lk(f->mu);
        f->stop = true;
    }
    f->cv.notify_all();
    {
        std::lock_guard<std::mutex> lk(f->pmu);
        f->stop = true;
    }
    f->pcv.notify_all();
    if (f->worker.joinable()) f->worker.join();
    for (auto &t : f->pool)
        if (t.joinable()) t.join();
    if (f->copy) (void)hipStreamSynchronize(f->copy);
    for (int b = 0; b < 2; ++b) {
        if (f->ev_assembled[b]) (void)hipEventSynchronize(f->ev_assembled[b]);
        (void)hipFree(f->d_code[b]);
        (void)hipFree(f->d_staged[b]);
    }
    (void)hipHostFree(f->h_idx);
    (void)hipHostFree(f->h_code);
    (void)hipHostFree(f->h_staged);
    for (hipEvent_t e : {f->ev_begin, f->ev_idx, f->ev_staged[0], f->ev_staged[1], f->ev_assembled[0],
                         f->ev_assembled[1]})
        if (e) (void)hipEventDestroy(e);
    if (f->copy) (void)hipStreamDestroy(f->copy);
    (void)hipGetLastError();
    delete f;
}

}  // namespace

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

    engram_plan_s *p = new (std::nothrow) engram_plan_s();
    if (!p) return ENGRAM_E_NOMEM;
    p->cfg = c;
    p->n_tables = n_tables;
    p->emb_dim = n_tables * c.head_dim;
    p->elem = elem;
    p->hc.n_tables = n_tables;
    p->hc.vocab = c.vocab;
    p->hc.vocab_comp = c.vocab_comp;
    for (int t = 0; t < n_tables; ++t) {
        p->hc.seed[t] = host_mix64(c.hash_seed + (uint64_t)(t + 1) * 0x9E3779B97F4A7C15ull);
        p->hc.rows[t] = c.table_rows[t];
        p->hc.magic[t] = UINT64_MAX / c.table_rows[t];
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

// ---------------------------------------------------------------- host-resident tables

engram_status engram_host_alloc(size_t bytes, void **ptr) {
    if (!ptr) return ENGRAM_E_INVALID_ARG;
    *ptr = nullptr;
    if (bytes == 0) return ENGRAM_E_INVALID_ARG;
    // mapped into every device's address space; non-coherent, so the GPU may
    // keep what it reads in its caches (the tables are read-only while used)
    if (hipHostMalloc(ptr, bytes, hipHostMallocMapped | hipHostMallocNonCoherent) != hipSuccess) {
        (void)hipGetLastError();
        *ptr = nullptr;
        return ENGRAM_E_NOMEM;
    }
    return ENGRAM_OK;
}

engram_status engram_host_free(void *ptr) {
    if (!ptr) return ENGRAM_OK;
    return hipHostFree(ptr) == hipSuccess ? ENGRAM_OK : ENGRAM_E_DEVICE;
}

namespace {
constexpr uint32_t kMaxCacheSlots = 1u << 28;

bool valid_cache(const engram_row_cache *c) {
    if (!c || c->capacity == 0) return true;
    return c->keys && c->rows && aligned16(c->keys) && aligned16(c->rows) && c->capacity <= kMaxCacheSlots &&
           (c->capacity & (c->capacity - 1u)) == 0;
}
}  // namespace

engram_status engram_cache_build(engram_plan p, const uint32_t *d_hot, int32_t n_hot, const void *const *table_ptrs,
                                 const engram_row_cache *cache, hipStream_t stream) {
    if (!p || !table_ptrs || !cache || cache->capacity == 0 || !valid_cache(cache)) return ENGRAM_E_INVALID_ARG;
    if (n_hot < 0 || (n_hot > 0 && !d_hot) || 2 * (int64_t)n_hot > (int64_t)cache->capacity)
        return ENGRAM_E_INVALID_ARG;
    for (int t = 0; t < p->n_tables; ++t)
        if (!table_ptrs[t] || !aligned16(table_ptrs[t])) return ENGRAM_E_INVALID_ARG;
    const GatherConsts gc = gather_consts(*p, table_ptrs);
    {
        Launch l(*p, ENGRAM_K_GATHER, stream);
        launch_cache_build(gc, cache->capacity, d_hot, n_hot, cache->keys, cache->rows, stream);
    }
    return last_launch_status();
}

engram_status engram_gather_cached(engram_plan p, const uint32_t *d_idx, int64_t n_tokens,
                                   const void *const *table_ptrs, const engram_row_cache *cache, void *d_emb,
                                   int32_t max_workgroups, hipStream_t stream) {
    engram_status st = check_gather_args(p, d_idx, n_tokens, table_ptrs, d_emb);
    if (st != ENGRAM_OK) return st;
    if (!valid_cache(cache) || max_workgroups < 0) return ENGRAM_E_INVALID_ARG;
    const GatherConsts gc = gather_consts(*p, table_ptrs);
    const uint32_t capacity = cache ? cache->capacity : 0u;
    {
        Launch l(*p, ENGRAM_K_GATHER, stream);
        launch_cached_gather(gc, capacity, d_idx, n_tokens, capacity ? cache->keys : nullptr,
                             capacity ? cache->rows : nullptr, d_emb, max_workgroups, stream);
    }
    return last_launch_status();
}

engram_status engram_gate_fuse(engram_plan p, const void *d_emb, const void *d_h, int32_t batch,
                               int32_t seqlen, const engram_weights *w, float *d_conv_state,
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
                             const engram_weights *w, float *d_conv_state, void *d_out,
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

// ---------------------------------------------------------------- backward

namespace {

struct BwdLayout {
    size_t E, KV, stats, dalpha, dconv, dg, dkv, wt, et, dkvt, demb, keys_in, keys_out, vals_in, vals_out, head,
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
    L.stats = take((size_t)(4 * Br * n_tok * 4));
    L.dalpha = take((size_t)(Br * L.n_stripes * n_tok * 4));
    L.dconv = take((size_t)L.conv_blocks * (size_t)(d * p.cfg.conv_kernel * 4));
    L.dg = take((size_t)(2 * Br * L.gate_chunks * d * 4));
    L.dkv = take((size_t)(n_tok * N * 2));
    L.wt = take((size_t)(De * N * 2));
    L.et = take((size_t)(De * n_pad * 2));
    L.dkvt = take((size_t)(N * n_pad * 2));
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
    uint16_t *wt = reinterpret_cast<uint16_t *>(base + L.wt);
    uint16_t *et = reinterpret_cast<uint16_t *>(base + L.et);
    uint16_t *dkvt = reinterpret_cast<uint16_t *>(base + L.dkvt);
    float *demb = reinterpret_cast<float *>(base + L.demb);
    engram_plan_s &P = *p;

    // retrieval again: E of the chunk
    st = do_gather(P, d_idx, n_tok, table_ptrs, E, stream);
    if (st != ENGRAM_OK) return st;
    // k of every branch and v, fp32
    {
        ProjArgs pa{};
        pa.emb = E;
        for (int m = 0; m <= kMaxBranches; ++m) pa.w[m] = m < Br ? w->w_k[m] : w->w_v;
        pa.n_tok = n_tok;
        pa.K = De;
        pa.d = d;
        pa.n_mats = Br + 1;
        pa.n_branches = Br;
        pa.out_f32 = KV;
        pa.out_ld = N;
        pa.n_rows = (int32_t)N;
        Launch l(P, ENGRAM_K_BWD_GEMM, stream);
        launch_proj_plain_bf16(pa, stream);
    }
    if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;

    BwdArgs ba{};
    ba.h = d_h;
    ba.dout = d_dout;
    ba.dh = d_dh;
    ba.kv = KV;
    ba.kv_ld = N;
    ba.stats = reinterpret_cast<float *>(base + L.stats);
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
        // backward, the small gradients' reductions and the operand transposes
        Launch l(P, ENGRAM_K_BWD_FUSE, stream);
        launch_bwd_gate_stats(ba, stream);
        launch_bwd_conv(ba, stream);
        launch_bwd_gate(ba, stream);
        float *part = reinterpret_cast<float *>(base + L.sum_part);
        launch_bwd_sum_rows(ba.dg_part, Br, L.gate_chunks, d, part, g->dgamma_h, stream);
        launch_bwd_sum_rows(ba.dg_part + (int64_t)Br * L.gate_chunks * d, Br, L.gate_chunks, d, part, g->dgamma_k,
                            stream);
        launch_bwd_sum_rows(ba.dconv_part, 1, L.conv_blocks, (int64_t)d * kc, part, g->dconv_w, stream);
        for (int m = 0; m <= Br; ++m)
            launch_bwd_transpose(static_cast<const uint16_t *>(m < Br ? w->w_k[m] : w->w_v), d, De, De,
                                 wt + (int64_t)m * d, N, d, stream);
        launch_bwd_transpose(static_cast<const uint16_t *>(E), n_tok, De, De, et, L.n_pad, L.n_pad, stream);
        launch_bwd_transpose(dkv, n_tok, N, N, dkvt, L.n_pad, L.n_pad, stream);
    }
    if (last_launch_status() != ENGRAM_OK) return ENGRAM_E_DEVICE;
    {
        // dE = [dk | dv] [W_k; W_v] and dW = [dk | dv]^T E on the MFMA loop
        Launch l(P, ENGRAM_K_BWD_GEMM, stream);
        ProjArgs pe{};
        pe.emb = dkv;
        for (int m = 0; m <= kMaxBranches; ++m) pe.w[m] = wt;
        pe.n_tok = n_tok;
        pe.K = (int32_t)N;
        pe.d = De;
        pe.n_mats = 1;
        pe.out_f32 = demb;
        pe.out_ld = De;
        pe.n_rows = De;
        launch_proj_plain_bf16(pe, stream);
        // dW contracts over every token: few output tiles, so K is split
        // until the chip is full and the partial results summed in order
        ProjArgs pw{};
        pw.emb = dkvt;
        for (int m = 0; m <= kMaxBranches; ++m) pw.w[m] = et;
        pw.n_tok = N;
        pw.K = (int32_t)(L.n_pad / L.dw_splits);
        pw.k_ld = (int32_t)L.n_pad;
        pw.d = De;
        pw.n_mats = 1;
        pw.out_f32 = L.dw_splits > 1 ? reinterpret_cast<float *>(base + L.dw_part) : g->dw;
        pw.out_ld = De;
        pw.out_split = N * De;
        pw.n_rows = De;
        launch_proj_plain_bf16(pw, stream, L.dw_splits);
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
    p->prof_max = max_launches;
    p->prof_used = 0;
    p->prof_dropped = 0;
    p->prof_on = true;
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

engram_status engram_prefetcher_create(engram_plan p, const void *const *host_tables, const engram_row_cache *cache,
                                       int64_t max_tokens, int32_t n_threads, engram_prefetcher *out) {
    if (!out) return ENGRAM_E_INVALID_ARG;
    *out = nullptr;
    if (!p || !host_tables || max_tokens <= 0 || n_threads < 1 || n_threads > 256 || !valid_cache(cache))
        return ENGRAM_E_INVALID_ARG;
    for (int t = 0; t < p->n_tables; ++t)
        if (!host_tables[t] || !aligned16(host_tables[t])) return ENGRAM_E_INVALID_ARG;
    const int64_t n_pairs = max_tokens * p->n_tables;
    if (n_pairs >= ((int64_t)1 << 31)) return ENGRAM_E_UNSUPPORTED;
    engram_prefetcher_s *f = new (std::nothrow) engram_prefetcher_s;
    if (!f) return ENGRAM_E_NOMEM;
    f->plan = p;
    f->gc = gather_consts(*p, host_tables);
    f->n_tables = p->n_tables;
    for (int t = 0; t < p->n_tables; ++t) {
        f->tables[t] = static_cast<const char *>(host_tables[t]);
        f->last_row[t] = p->cfg.table_rows[t] - 1;
    }
    if (cache) f->cache = *cache;
    f->max_tok = max_tokens;
    f->n_threads = n_threads;
    f->row_bytes = (size_t)p->cfg.head_dim * p->elem;
    f->terr.assign(n_threads, hipSuccess);
    f->tcount.assign(n_threads, 0u);
    bool ok = hipGetDevice(&f->dev) == hipSuccess;
    try {
        f->keys.assign((size_t)p->n_tables * f->cache.capacity, 0u);
    } catch (...) {
        ok = false;
    }
    // the cache is fixed while the prefetcher lives: its keys are read once
    if (ok && f->cache.capacity)
        ok = hipMemcpy(f->keys.data(), f->cache.keys, f->keys.size() * 4, hipMemcpyDeviceToHost) == hipSuccess;
    for (int b = 0; b < 2; ++b) {
        ok = ok && hipMalloc(&f->d_code[b], (size_t)n_pairs * 4) == hipSuccess;
        ok = ok && hipMalloc(&f->d_staged[b], (size_t)n_pairs * f->row_bytes) == hipSuccess;
    }
    ok = ok && hipHostMalloc(&f->h_idx, (size_t)n_pairs * 4, hipHostMallocDefault) == hipSuccess;
    ok = ok && hipHostMalloc(&f->h_code, (size_t)n_pairs * 4, hipHostMallocDefault) == hipSuccess;
    ok = ok && hipHostMalloc(&f->h_staged, (size_t)n_pairs * f->row_bytes, hipHostMallocDefault) == hipSuccess;
    ok = ok && hipStreamCreateWithFlags(&f->copy, hipStreamNonBlocking) == hipSuccess;
    for (hipEvent_t *e : {&f->ev_begin, &f->ev_idx, &f->ev_staged[0], &f->ev_staged[1], &f->ev_assembled[0],
                          &f->ev_assembled[1]})
        ok = ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        prefetcher_free(f);
        return ENGRAM_E_NOMEM;
    }
    try {
        for (int t = 1; t < n_threads; ++t) f->pool.emplace_back(pool_main, f, t);
        f->worker = std::thread(worker_main, f);
    } catch (...) {
        prefetcher_free(f);
        return ENGRAM_E_NOMEM;
    }
    *out = f;
    return ENGRAM_OK;
}

engram_status engram_prefetcher_destroy(engram_prefetcher f) {
    if (!f) return ENGRAM_E_INVALID_ARG;
    {
        // a job in flight ends first
        std::unique_lock<std::mutex> lk(f->mu);
        f->cv.wait(lk, [&] { return f->state != engram_prefetcher_s::LISTING; });
    }
    prefetcher_free(f);
    return ENGRAM_OK;
}

engram_status engram_prefetch_begin(engram_prefetcher f, const uint32_t *d_idx, int64_t n_tok, hipStream_t stream) {
    if (!f || !d_idx || !aligned16(d_idx) || n_tok <= 0 || n_tok > f->max_tok) return ENGRAM_E_INVALID_ARG;
    int set;
    {
        std::lock_guard<std::mutex> lk(f->mu);
        if (f->state != engram_prefetcher_s::IDLE) return ENGRAM_E_INVALID_ARG;  // a job is in flight
        set = (int)(f->job_count & 1u);
    }
    // the indices reach the host on the copy stream, after the work that
    // produced them on `stream`; no kernel is queued
    if (hipEventRecord(f->ev_begin, stream) != hipSuccess || hipStreamWaitEvent(f->copy, f->ev_begin, 0) != hipSuccess ||
        hipMemcpyAsync(f->h_idx, d_idx, (size_t)n_tok * f->n_tables * 4, hipMemcpyDeviceToHost, f->copy) != hipSuccess ||
        hipEventRecord(f->ev_idx, f->copy) != hipSuccess) {
        (void)hipGetLastError();
        return ENGRAM_E_DEVICE;
    }
    {
        std::lock_guard<std::mutex> lk(f->mu);
        f->job_tok = n_tok;
        f->job_set = set;
        ++f->job_count;
        f->state = engram_prefetcher_s::LISTING;
    }
    f->cv.notify_all();
    return ENGRAM_OK;
}

engram_status engram_prefetch_finish(engram_prefetcher f, void *d_emb, uint32_t *h_misses_out, hipStream_t stream) {
    if (!f || !d_emb || !aligned16(d_emb)) return ENGRAM_E_INVALID_ARG;
    int64_t n_tok;
    hipError_t e;
    uint32_t n_miss;
    int set;
    {
        std::unique_lock<std::mutex> lk(f->mu);
        if (f->state == engram_prefetcher_s::IDLE) return ENGRAM_E_INVALID_ARG;  // nothing begun
        f->cv.wait(lk, [&] { return f->state == engram_prefetcher_s::STAGED; });
        n_tok = f->job_tok;
        e = f->err;
        n_miss = f->job_misses;
        set = f->job_set;
        f->state = engram_prefetcher_s::IDLE;
    }
    if (h_misses_out) *h_misses_out = n_miss;
    if (e != hipSuccess) return ENGRAM_E_DEVICE;
    if (hipStreamWaitEvent(stream, f->ev_staged[set], 0) != hipSuccess) return ENGRAM_E_DEVICE;
    {
        Launch l(*f->plan, ENGRAM_K_GATHER, stream);
        launch_prefetch_assemble(f->gc, n_tok, f->d_code[set], f->cache.rows, f->d_staged[set], d_emb, stream);
    }
    if (last_launch_status() != ENGRAM_OK || hipEventRecord(f->ev_assembled[set], stream) != hipSuccess)
        return ENGRAM_E_DEVICE;
    f->assembled[set] = true;
    return ENGRAM_OK;
}

}  // extern "C"
