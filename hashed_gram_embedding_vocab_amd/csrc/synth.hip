// synth.hip -- synthetic embedding-table contents (test and benchmark input,
// not part of the Engram method).  Trained table rows are unavailable, so
// tables hold deterministic pseudo-random values: for table tau, row r,
// column c the Philox4x64-10 block at counter (r, c/4, tau, 0) and key
// (seed, 0) (Salmon, Moraes, Dror & Shaw, SC'11) gives four 64-bit words;
// word c%4 is split into four 16-bit fields whose sum S is an Irwin-Hall(4)
// variate, and the value is fp32(S - 131070) * 0x1.1bc77ap-21 (standard
// deviation 0.02), rounded to nearest-even bf16 for bf16 tables.  Filling on
// the device lets 200 GB of tables exist without a host copy.
#include "engram_internal.h"

namespace engram {
namespace {

__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t lo0 = 0xD2E7470EE14C6C93ull * c[0];
        const uint64_t hi0 = __umul64hi(0xD2E7470EE14C6C93ull, c[0]);
        const uint64_t lo1 = 0xCA5A826395121157ull * c[2];
        const uint64_t hi1 = __umul64hi(0xCA5A826395121157ull, c[2]);
        const uint64_t n0 = hi1 ^ c[1] ^ k0;
        const uint64_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
}

__device__ __forceinline__ float ih4_value(uint64_t w) {
    const int32_t s = (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) +
                      (int32_t)((w >> 32) & 0xFFFF) + (int32_t)(w >> 48);
    return __fmul_rn((float)(s - 131070), 0x1.1bc77ap-21f);
}

template <bool BF16>
__global__ __launch_bounds__(256) void synth_fill_kernel(uint64_t seed, int32_t tau, int64_t rows,
                                                         int32_t groups, void *table) {
    const int64_t total = rows * groups;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = g / groups;
        const int32_t q = (int32_t)(g - row * groups);
        uint64_t c[4] = {(uint64_t)row, (uint64_t)q, (uint64_t)tau, 0};
        philox4x64_10(c, seed, 0);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = ih4_value(c[i]);
        if constexpr (BF16) {
            // integer round-to-nearest-even: bit-exact whatever the FP mode register says
            u32x2_t p = {f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16), f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16)};
            reinterpret_cast<u32x2_t *>(table)[g] = p;
        } else {
            reinterpret_cast<f32x4_t *>(table)[g] = f32x4_t{v[0], v[1], v[2], v[3]};
        }
    }
}

}  // namespace

void launch_synth_fill(engram_dtype dt, uint64_t seed, int32_t tau, int64_t rows, int32_t head_dim,
                       void *table, hipStream_t s) {
    const int32_t groups = head_dim / 4;
    const int64_t total = rows * groups;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256 * 1024) blocks = 256 * 1024;
    if (dt == ENGRAM_BF16)
        launch_kernel(synth_fill_kernel<true>, dim3((unsigned)blocks), dim3(256), s, seed, tau,
                           rows, groups, table);
    else
        launch_kernel(synth_fill_kernel<false>, dim3((unsigned)blocks), dim3(256), s, seed, tau,
                           rows, groups, table);
}

}  // namespace engram
