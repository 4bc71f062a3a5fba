// hash_math.h -- the integer arithmetic of the multi-head n-gram hash, for
// both the kernels and the host (plan creation computes the per-table seeds
// and reduction constants with these same functions, and a CPU test checks
// the reduction against an exact 64-bit remainder).
//
// The pages ([club] 二.1(1), multi-head hashing into prime-sized tables) fix
// only that each head maps an n-gram deterministically to a slot of its own
// table; the mixer and the reduction below are this library's choice.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

// SplitMix64 output function (Steele, Lea & Flood 2014; Mix13 constants):
// the deterministic mixer of the multi-head n-gram hash.
__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

// Per-table seed of table tau: the tau-th output of SplitMix64 started at
// the plan's hash seed (its state advances by the golden-ratio increment).
__host__ __device__ __forceinline__ uint64_t table_seed(uint64_t hash_seed, int tau) {
    return mix64(hash_seed + (uint64_t)(tau + 1) * 0x9E3779B97F4A7C15ull);
}

// High 64 bits of a 64 x 64-bit product (one v_mad_u64_u32 chain on the GPU).
__host__ __device__ __forceinline__ uint64_t mulhi64(uint64_t a, uint64_t b) {
    return (uint64_t)(((unsigned __int128)a * b) >> 64);
}

// Reduction constant of a table with p rows: m = floor((2^64 - 1) / p).
__host__ __device__ __forceinline__ uint64_t mod_magic(uint32_t p) {
    return UINT64_MAX / p;
}

// z mod p for a 64-bit z and 32-bit p >= 1 without a hardware divide.  With
// m = floor((2^64-1)/p) = (2^64 - 1 - r0)/p, r0 = (2^64-1) mod p < p:
//   z*m/2^64 = z/p - z*(1 + r0)/(p*2^64) > z/p - 1   (as z < 2^64, 1 + r0 <= p),
// so q = floor(z*m/2^64) is floor(z/p) or one below it and z - q*p < 2p.  The
// second subtraction is never taken; it is kept so the bound needs no proof
// at the call site.
__host__ __device__ __forceinline__ uint32_t mod_prime(uint64_t z, uint32_t p, uint64_t m) {
    const uint64_t q = mulhi64(z, m);
    uint64_t r = z - q * (uint64_t)p;
    if (r >= p) r -= p;
    if (r >= p) r -= p;
    return (uint32_t)r;
}

}  // namespace engram
