// api_noalloc.hip -- engram_forward_noalloc (include/engram.h): the forward
// pass for callers that cannot allocate device memory, with its workspace in
// a scratch array the library holds on every GPU it runs on.
//
// The array is a file-scope __device__ variable, so each GPU gets its own copy
// when the code object is loaded there.  In host code its name is only a
// host-side stand-in, never a device address: the device address comes from
// hipGetSymbolAddress, once per device (with that device current), and is kept
// in device_scratch below; only that pointer is ever handed to a kernel.
//
// engram_forward writes every workspace region it reads within the same call
// (slots, E, gate partials, gates, seam rows, state staging), so nothing in the
// array has to start at zero and a call never sees the previous call's data.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "engram.h"

namespace {

constexpr size_t kScratchBytes = (size_t)ENGRAM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};

// The current device's copy of the array (looked up on the first call on each
// device), or null if the runtime cannot give its address.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

engram_status engram_forward_noalloc(engram_plan p, const int32_t *d_tokens, int32_t batch, int32_t seqlen,
                                     const int32_t *d_comp_map, int32_t *d_prev_ctx,
                                     const void *const *table_ptrs, const void *d_h, const engram_weights *w,
                                     void *d_conv_state, void *d_out, float *d_alpha, uint32_t flags,
                                     uint32_t *d_bad_tokens, hipStream_t stream) {
    if (!p || batch <= 0 || seqlen <= 0) return ENGRAM_E_INVALID_ARG;
    const size_t need = engram_workspace_size(p, batch, seqlen);
    if (need == 0) return ENGRAM_E_INVALID_ARG;
    if (need > kScratchBytes) return ENGRAM_E_UNSUPPORTED;
    void *ws = device_scratch();
    if (!ws) return ENGRAM_E_DEVICE;
    return engram_forward(p, d_tokens, batch, seqlen, d_comp_map, d_prev_ctx, table_ptrs, d_h, w, d_conv_state,
                          d_out, d_alpha, flags, ws, kScratchBytes, d_bad_tokens, stream);
}

}  // extern "C"
