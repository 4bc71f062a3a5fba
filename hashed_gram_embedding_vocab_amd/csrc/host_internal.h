// host_internal.h -- what the host side of the C ABI shares between its
// files (api.cpp: plans, retrieval and fusion; api_backward.cpp: the
// backward; api_offload.cpp: host-resident tables and the prefetcher): the
// plan, the profiling scope of a launch, argument checks and the row gather.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "engram.h"
#include "engram_internal.h"

struct engram_plan_s {
    engram_config cfg;
    int32_t n_tables = 0;
    int32_t emb_dim = 0;    // D_e
    int32_t elem = 0;       // bytes per element of the plan dtype
    bool state_bf16 = false;  // the carried conv state is bf16
    engram::HashConsts hc{};
    // profiling
    bool prof_on = false;
    uint32_t prof_mask = 0;
    int32_t prof_max = 0;
    int32_t prof_used = 0;
    int64_t prof_dropped = 0;
    int32_t prof_every = 1;                 // time one launch in prof_every of each kind
    int64_t prof_seen[ENGRAM_K_COUNT] = {};  // launches of each selected kind since profiling began
    std::vector<hipEvent_t> prof_ev;
    std::vector<int32_t> prof_kind;
};

namespace engram {
namespace host {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// One timed library launch while profiling is on: hands a pair of the
// plan's events to the kernel launches in its scope (see launch_kernel).
struct Launch {
    engram_plan_s &p;
    int32_t slot = -1;
    Launch(engram_plan_s &pl, int32_t kind, hipStream_t) : p(pl) {
        if (!p.prof_on || !((p.prof_mask >> kind) & 1u)) return;
        if (p.prof_seen[kind]++ % p.prof_every != 0) return;
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

inline engram_status last_launch_status() {
    return hipGetLastError() == hipSuccess ? ENGRAM_OK : ENGRAM_E_DEVICE;
}

// Arguments of a row gather (engram_gather and the calls built on it).
engram_status check_gather_args(const engram_plan_s *p, const uint32_t *idx, int64_t n_tok,
                                const void *const *tables, const void *emb);
// The gather kernels' view of a plan's tables.
GatherConsts gather_consts(const engram_plan_s &p, const void *const *tables);
// E[t] = concat of the tables' rows idx[t][.], one launch (timed as ENGRAM_K_GATHER).
engram_status do_gather(engram_plan_s &p, const uint32_t *idx, int64_t n_tok, const void *const *tables,
                        void *emb, hipStream_t s);

}  // namespace host
}  // namespace engram
