// stream_probe.hip -- measurement helpers, not part of the method: a plain
// streaming read and a plain streaming copy of a device buffer, the ceilings
// that the retrieval kernels' bytes per second are set against, and the
// known byte counts that scale the FETCH_SIZE / WRITE_SIZE counters.
//
// A workgroup walks the buffer in slabs of 256 threads x U 16-byte chunks
// (consecutive lanes read consecutive chunks, so every wave reads whole
// 1 KB runs); all U loads of a slab are issued before any is consumed.  The
// grid is a fixed number of workgroups per CU that stride over the buffer.
// The read probe folds what it loads into one value per thread and stores it
// only if it equals a constant no input is built to produce, so the loads
// cannot be dropped and no bytes are written.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;

template <int U, bool NT>
__device__ __forceinline__ u32x4_t load_chunk(const u32x4_t *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t *__restrict__ src, int64_t chunks,
                                                               u32x4_t *__restrict__ sink) {
    const int64_t slab = (int64_t)kThreads * U;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int64_t base = (int64_t)blockIdx.x * slab; base < chunks; base += (int64_t)gridDim.x * slab) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = base + u * kThreads + threadIdx.x;
            v[u] = load_chunk<U, NT>(src + (c < chunks ? c : chunks - 1));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0xBF58476Du && acc.w == 0x1CE4E5B9u)
        sink[0] = acc;
}

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const u32x4_t *__restrict__ src, int64_t chunks,
                                                               u32x4_t *__restrict__ dst) {
    const int64_t slab = (int64_t)kThreads * U;
    for (int64_t base = (int64_t)blockIdx.x * slab; base < chunks; base += (int64_t)gridDim.x * slab) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = base + u * kThreads + threadIdx.x;
            v[u] = load_chunk<U, NT>(src + (c < chunks ? c : chunks - 1));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = base + u * kThreads + threadIdx.x;
            if (c < chunks) {
                if constexpr (NT) __builtin_nontemporal_store(v[u], dst + c);
                else dst[c] = v[u];
            }
        }
    }
}

template <int U, bool NT>
void launch_u(int mode, const void *src, void *dst, int64_t chunks, int blocks, hipStream_t s) {
    if (mode == 0)
        launch_kernel(stream_read_kernel<U, NT>, dim3((unsigned)blocks), dim3(kThreads), s,
                      static_cast<const u32x4_t *>(src), chunks, static_cast<u32x4_t *>(dst));
    else
        launch_kernel(stream_copy_kernel<U, NT>, dim3((unsigned)blocks), dim3(kThreads), s,
                      static_cast<const u32x4_t *>(src), chunks, static_cast<u32x4_t *>(dst));
}

}  // namespace

bool launch_stream_probe(int mode, bool nontemporal, int unroll, const void *src, void *dst, int64_t bytes,
                         int blocks, hipStream_t s) {
    const int64_t chunks = bytes / 16;
#define ENGRAM_PROBE_CASE(U)                                                        \
    case U:                                                                          \
        if (nontemporal) launch_u<U, true>(mode, src, dst, chunks, blocks, s);       \
        else launch_u<U, false>(mode, src, dst, chunks, blocks, s);                  \
        return true;
    switch (unroll) {
        ENGRAM_PROBE_CASE(4)
        ENGRAM_PROBE_CASE(8)
        ENGRAM_PROBE_CASE(16)
        default: return false;
    }
#undef ENGRAM_PROBE_CASE
}

}  // namespace engram
