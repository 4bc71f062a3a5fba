// Host-side check of the kernels' table-slot reduction (hash_math.h):
// mod_prime(z, p, mod_magic(p)) must equal the exact remainder z % p.
//
//   mod_prime_check N_RANDOM p1 p2 ...
//
// For every prime p given: z at the ends of the 64-bit range, at 0..3,
// around every power of two, and k*p - 1, k*p, k*p + 1 for k at the ends of
// [1, floor((2^64-1)/p)] and around every power of two in that range; then
// N_RANDOM pseudo-random z (an xorshift64* stream, any source of spread-out
// 64-bit values serves).  Prints the number of values checked and exits 1
// with the first mismatch, if any.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "hash_math.h"

static uint64_t n_checked = 0;

static bool check(uint64_t z, uint32_t p, uint64_t m) {
    ++n_checked;
    const uint32_t got = engram::mod_prime(z, p, m);
    const uint64_t want = z % p;
    if (got != want) {
        std::printf("MISMATCH z=%llu p=%u got=%u want=%llu\n", (unsigned long long)z, p, got,
                    (unsigned long long)want);
        return false;
    }
    return true;
}

int main(int argc, char **argv) {
    if (argc < 3) {
        std::fprintf(stderr, "usage: %s N_RANDOM p1 [p2 ...]\n", argv[0]);
        return 2;
    }
    const uint64_t n_random = std::strtoull(argv[1], nullptr, 10);
    uint64_t x = 0x2545F4914F6CDD1Dull;
    for (int a = 2; a < argc; ++a) {
        const uint32_t p = (uint32_t)std::strtoul(argv[a], nullptr, 10);
        if (p == 0) return 2;
        const uint64_t m = engram::mod_magic(p);
        bool ok = true;
        const uint64_t ends[] = {0, 1, 2, 3, UINT64_MAX, UINT64_MAX - 1, UINT64_MAX - 2, p - 1ull, p, p + 1ull};
        for (uint64_t z : ends) ok &= check(z, p, m);
        for (int b = 1; b < 64; ++b) {
            const uint64_t z = 1ull << b;
            ok &= check(z - 1, p, m) & check(z, p, m) & check(z + 1, p, m);
        }
        const uint64_t kmax = UINT64_MAX / p;
        uint64_t ks[200];
        int nk = 0;
        ks[nk++] = 1; ks[nk++] = 2; ks[nk++] = kmax; ks[nk++] = kmax - 1;
        for (int b = 1; b < 64 && (1ull << b) <= kmax; ++b) {
            ks[nk++] = (1ull << b) - 1;
            ks[nk++] = 1ull << b;
        }
        for (int i = 0; i < nk; ++i) {
            const uint64_t kp = ks[i] * (uint64_t)p;  // <= kmax * p <= 2^64 - 1
            ok &= check(kp - 1, p, m) & check(kp, p, m);
            if (kp != UINT64_MAX) ok &= check(kp + 1, p, m);
        }
        for (uint64_t i = 0; i < n_random && ok; ++i) {
            x ^= x >> 12; x ^= x << 25; x ^= x >> 27;
            ok &= check(x * 0x2545F4914F6CDD1Dull, p, m);
        }
        if (!ok) return 1;
    }
    std::printf("checked %llu\n", (unsigned long long)n_checked);
    return 0;
}
