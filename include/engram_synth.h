/*
 * engram_synth.h -- harness entry points for tests and benchmarks, not part
 * of the Engram method:
 *   - synthetic embedding-table contents: trained table rows are not
 *     available, so tables are filled on the device with deterministic
 *     pseudo-random values that any independent implementation of the same
 *     published generator reproduces bit for bit;
 *   - a plain streaming read and copy of a device buffer: the bandwidth
 *     ceilings the retrieval kernels are compared with, and buffers of known
 *     size for scaling hardware traffic counters.
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

/*
 * One streaming pass over a device buffer.
 *   mode     0: read `bytes` from d_src (d_dst: a 16-byte sink that no input
 *               built here makes the kernel write); 1: copy `bytes` from
 *               d_src to d_dst
 *   flags    ENGRAM_PROBE_NONTEMPORAL: nontemporal loads (and stores)
 *   unroll   16-byte chunks in flight per thread: 4, 8 or 16
 *   blocks   workgroups of 256 threads that stride over the buffer, 1..2^20
 *   bytes    > 0, a multiple of 16; both pointers 16-byte aligned, caller-owned
 * Asynchronous on `stream`; ENGRAM_E_INVALID_ARG on bad arguments (nothing
 * launched), ENGRAM_E_DEVICE if the launch fails.
 */
enum { ENGRAM_PROBE_NONTEMPORAL = 1u << 0 };
ENGRAM_API engram_status engram_probe_stream(int32_t mode, uint32_t flags, int32_t unroll, int32_t blocks,
                                             const void *d_src, void *d_dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_SYNTH_H */
