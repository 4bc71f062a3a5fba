/*
 * engram_synth.h -- synthetic embedding-table contents for tests and
 * benchmarks.  Not part of the Engram method: trained table rows are not
 * available, so tables are filled on the device with deterministic
 * pseudo-random values that any independent implementation of the same
 * published generator reproduces bit for bit.
 */
#ifndef ENGRAM_SYNTH_H
#define ENGRAM_SYNTH_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "engram.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Fill table tau ([rows][head_dim] row-major, dtype ENGRAM_F32 or
 * ENGRAM_BF16) on the device.  Element (r, c) is built from the Philox4x64-10
 * block (Salmon, Moraes, Dror & Shaw, SC'11) at counter (r, c/4, tau, 0) with
 * key (seed, 0): word c%4 is cut into four 16-bit fields, their sum S is
 * Irwin-Hall distributed, and the value is fp32(S - 131070) * 0x1.1bc77ap-21
 * (mean 0, standard deviation 0.02), rounded to nearest-even for bf16.
 *   d_table  caller-owned device buffer, 16-byte aligned
 *   head_dim multiple of 4
 * Asynchronous on `stream`; returns ENGRAM_E_INVALID_ARG on bad arguments.
 */
ENGRAM_API engram_status engram_synth_fill_table(int32_t dtype, uint64_t seed, int32_t tau, int64_t rows,
                                      int32_t head_dim, void *d_table, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_SYNTH_H */
