// noalloc.hip -- hla_forward_noalloc: hla_forward with its workspace (the
// segment summaries and up-sweep nodes of the scan, and third order's Y) in
// a fixed device array of this library instead of a caller buffer, for
// callers that cannot allocate device memory.
//
// The array below is a device symbol: in host code its name is a host-side
// stand-in, not a device address.  Its address on each device is looked up
// once, with that device current, and only that address is handed to the
// kernels.  Each device holds its own copy for the life of the process.
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/hla.h"
#include "launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[HLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];   // device address of `scratch`, per device id

// The address of `scratch` on the current device, looked up on the first
// call for that device.
hla_status scratch_on_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HLA_ERR_DEVICE;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return HLA_ERR_DEVICE;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return HLA_OK;
}

}  // namespace

extern "C" hla_status hla_forward_noalloc(const void *q, const void *k, const void *v, void *o,
                                          int B, int H, int n, int d, int dv, int dtype,
                                          int variant, const float *gamma_host, int chunk,
                                          int seg_chunks, const float *state_in,
                                          float *state_out, void *stream) {
    size_t need = 0;
    hla_status st = hla::forward_validate(q, k, v, o, B, H, n, d, dv, dtype, variant, gamma_host,
                                          chunk, seg_chunks, state_in, state_out, &need);
    if (st != HLA_OK) return st;
    if (need > HLA_NOALLOC_SCRATCH_BYTES) return HLA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_on_current_device(&ws);
        if (st != HLA_OK) return st;
    }
    // the kernels write every part of the workspace they read, so the
    // array's contents from an earlier call need no clearing
    return hla_forward(q, k, v, o, B, H, n, d, dv, dtype, variant, gamma_host, chunk, seg_chunks,
                       state_in, state_out, ws, need > 0 ? (size_t)HLA_NOALLOC_SCRATCH_BYTES : 0,
                       stream);
}
