// api_offload.cpp -- host side of the host-resident tables (include/engram.h):
// pinned host allocation, the HBM hot-row cache and its gather, and the
// host-gather prefetcher (its worker and pool threads).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "host_internal.h"

using namespace engram;
using namespace engram::host;

namespace {
constexpr uint32_t kMaxCacheSlots = 1u << 28;

bool valid_cache(const engram_row_cache *c) {
    if (!c || c->capacity == 0) return true;
    return c->keys && c->rows && aligned16(c->keys) && aligned16(c->rows) && c->capacity <= kMaxCacheSlots &&
           (c->capacity & (c->capacity - 1u)) == 0;
}
}  // namespace

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
