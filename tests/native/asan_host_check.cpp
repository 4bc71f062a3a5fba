// The host side of libengram's C ABI under AddressSanitizer, on a machine
// without a GPU: plan creation and destruction over valid and invalid
// configurations, the workspace sizes, status strings, and every entry point
// called with arguments its host-side validation rejects before anything
// reaches a device (fake device pointers are never dereferenced).  Built with
// the sanitizer on host code only; prints "ok" and exits 0 when every call
// returned the status expected.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "engram.h"
#include "engram_synth.h"

static int fails = 0;
#define EXPECT(expr, want)                                                                    \
    do {                                                                                      \
        const int got_ = (int)(expr);                                                         \
        if (got_ != (int)(want)) {                                                            \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, \
                         (int)(want));                                                        \
            ++fails;                                                                          \
        }                                                                                     \
    } while (0)

static engram_config base_config(engram_dtype dt) {
    engram_config c;
    std::memset(&c, 0, sizeof(c));
    c.vocab = 1000;
    c.vocab_comp = 770;
    c.n_orders = 2;
    c.orders[0] = 2;
    c.orders[1] = 3;
    c.heads = 8;
    c.head_dim = 64;
    for (int t = 0; t < 16; ++t) c.table_rows[t] = 10007u - 2u * t;
    c.hash_seed = 1;
    c.d_model = 512;
    c.n_branches = 2;
    c.conv_kernel = 4;
    c.conv_mode = ENGRAM_CONV_LINEAR;
    c.rms_eps = 1e-6f;
    c.dtype = dt;
    c.state_dtype = ENGRAM_F32;
    return c;
}

int main() {
    for (int s = -1; s < 7; ++s) EXPECT(engram_status_string((engram_status)s) != nullptr, 1);

    // plans: valid ones and one bad field at a time
    std::vector<engram_config> bad;
    for (int k = 0; k < 12; ++k) {
        engram_config c = base_config(ENGRAM_BF16);
        switch (k) {
            case 0: c.vocab_comp = 1 << 21; break;
            case 1: c.heads = 17; break;
            case 2: c.head_dim = 30; break;
            case 3: c.d_model = 100; break;
            case 4: c.n_branches = 5; break;
            case 5: c.conv_kernel = 5; break;
            case 6: c.conv_mode = 7; break;
            case 7: c.orders[1] = 4; break;
            case 8: c.table_rows[5] = 0; break;
            case 9: c.rms_eps = -1.f; break;
            case 10: c.state_dtype = (engram_dtype)7; break;
            case 11: c.dtype = ENGRAM_F32; c.state_dtype = ENGRAM_BF16; break;
        }
        bad.push_back(c);
    }
    for (const engram_config &c : bad) {
        engram_plan p = nullptr;
        EXPECT(engram_plan_create(&c, &p), ENGRAM_E_INVALID_ARG);
        EXPECT(p == nullptr, 1);
    }
    EXPECT(engram_plan_create(nullptr, nullptr), ENGRAM_E_INVALID_ARG);
    EXPECT(engram_plan_destroy(nullptr), ENGRAM_E_INVALID_ARG);

    const engram_dtype dts[2] = {ENGRAM_F32, ENGRAM_BF16};
    for (engram_dtype dt : dts) {
        engram_config c = base_config(dt);
        if (dt == ENGRAM_BF16) c.state_dtype = ENGRAM_BF16;
        engram_plan p = nullptr;
        EXPECT(engram_plan_create(&c, &p), ENGRAM_OK);
        const int shapes[5][2] = {{1, 1}, {3, 77}, {8, 4096}, {256, 1}, {1, 32768}};
        for (auto &sh : shapes) {
            EXPECT(engram_workspace_size(p, sh[0], sh[1]) > 0, 1);
            (void)engram_backward_workspace_size(p, sh[0], sh[1]);
        }
        EXPECT(engram_workspace_size(p, 0, 5), 0);
        EXPECT(engram_workspace_size(nullptr, 1, 1), 0);

        // entry points with arguments rejected before any device work
        const uintptr_t F = 0x10000;  // a 16-byte-aligned address never dereferenced
        void *fake = reinterpret_cast<void *>(F);
        void *odd = reinterpret_cast<void *>(F + 4);
        const void *tabs[32];
        for (auto &t : tabs) t = fake;
        engram_weights w;
        std::memset(&w, 0, sizeof(w));
        int32_t *ti = static_cast<int32_t *>(fake);
        uint32_t *tu = static_cast<uint32_t *>(fake);
        EXPECT(engram_hash(nullptr, ti, 1, 1, ti, nullptr, tu, nullptr, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_hash(p, ti, 0, 1, ti, nullptr, tu, nullptr, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_hash(p, static_cast<int32_t *>(odd), 1, 1, ti, nullptr, tu, nullptr, nullptr),
               ENGRAM_E_INVALID_ARG);
        EXPECT(engram_gather(p, tu, 0, tabs, fake, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_gather(p, tu, 5, nullptr, fake, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_gather(p, tu, 5, tabs, odd, nullptr), ENGRAM_E_INVALID_ARG);
        // null weights inside the struct
        EXPECT(engram_gate_fuse(p, fake, fake, 2, 9, &w, nullptr, fake, nullptr, 0, fake, 1u << 30, nullptr),
               ENGRAM_E_INVALID_ARG);
        EXPECT(engram_forward(p, ti, 2, 9, ti, nullptr, tabs, fake, &w, nullptr, fake, nullptr, 0, fake, 1u << 30,
                              nullptr, nullptr),
               ENGRAM_E_INVALID_ARG);
        EXPECT(engram_forward(p, ti, 2, 9, ti, nullptr, tabs, fake, &w, nullptr, fake, nullptr, 0, nullptr, 0,
                              nullptr, nullptr),
               ENGRAM_E_INVALID_ARG);
        // beyond the no-allocation scratch: rejected before any device call
        EXPECT(engram_forward_noalloc(p, ti, 64, 4096, ti, nullptr, tabs, fake, &w, nullptr, fake, nullptr, 0,
                                      nullptr, nullptr),
               ENGRAM_E_UNSUPPORTED);
        EXPECT(engram_forward_noalloc(nullptr, ti, 1, 1, ti, nullptr, tabs, fake, &w, nullptr, fake, nullptr, 0,
                                      nullptr, nullptr),
               ENGRAM_E_INVALID_ARG);
        EXPECT(engram_retrieve(p, ti, 0, 4, ti, nullptr, tabs, fake, nullptr, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_retrieve(p, ti, 2, 4, ti, nullptr, tabs, odd, nullptr, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_retrieve(nullptr, ti, 2, 4, ti, nullptr, tabs, fake, nullptr, nullptr),
               ENGRAM_E_INVALID_ARG);
        engram_grads g;
        std::memset(&g, 0, sizeof(g));
        EXPECT(engram_backward(p, tu, tabs, fake, &w, fake, 2, 9, 0, fake, &g, fake, 0, nullptr),
               dt == ENGRAM_BF16 ? ENGRAM_E_INVALID_ARG : ENGRAM_E_UNSUPPORTED);
        engram_row_cache rc;
        std::memset(&rc, 0, sizeof(rc));
        rc.capacity = 3;  // not a power of two
        EXPECT(engram_cache_build(p, tu, 4, tabs, &rc, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_gather_cached(p, tu, 0, tabs, &rc, fake, 0, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_prefetcher_create(p, nullptr, nullptr, 10, 2, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_prefetcher_destroy(nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_prefetch_begin(nullptr, tu, 1, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_prefetch_finish(nullptr, fake, nullptr, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_profile_begin(p, 0, 0), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_profile_begin(p, 16, 1u << 20), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_profile_every(p, 0), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_profile_end(p, nullptr), ENGRAM_E_INVALID_ARG);
        EXPECT(engram_plan_destroy(p), ENGRAM_OK);
    }
    void *fake = reinterpret_cast<void *>(0x10000);
    EXPECT(engram_synth_fill_table(7, 1, 0, 10, 8, fake, nullptr), ENGRAM_E_INVALID_ARG);
    EXPECT(engram_synth_fill_table(ENGRAM_BF16, 1, 0, 10, 6, fake, nullptr), ENGRAM_E_INVALID_ARG);
    EXPECT(engram_probe_stream(2, 0, 8, 64, fake, fake, 4096, nullptr), ENGRAM_E_INVALID_ARG);
    EXPECT(engram_probe_stream(0, 0, 8, 64, fake, fake, 4095, nullptr), ENGRAM_E_INVALID_ARG);
    EXPECT(engram_host_free(nullptr), ENGRAM_OK);  // NULL is accepted
    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
