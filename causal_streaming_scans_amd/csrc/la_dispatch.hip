// la_dispatch.hip -- instances of the chunked first-order linear-attention
// kernels (la_kernels.h) and their run-time lookup.
#include "la_kernels.h"
#include "launch.h"

namespace hla {

template <typename T, int D>
hipError_t launch_la(const LaParams &p, hipStream_t s) {
    constexpr int C = kLaChunk;
    if (p.nseg > 1) {
        hipLaunchKernelGGL((la_summary_kernel<T, D, C>), dim3((p.nseg - 1) * p.BH),
                           dim3(LaCfg<T, D, C>::NT), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((la_forward_kernel<T, D, C>), dim3(p.nseg * p.BH), dim3(LaCfg<T, D, C>::NT),
                       0, s, p);
    return hipGetLastError();
}

bool lookup_la(int dtype, int d, LaLaunch *out) {
    if (dtype == 0) {
        switch (d) {
            case 16: *out = launch_la<float, 16>; return true;
            case 32: *out = launch_la<float, 32>; return true;
            case 64: *out = launch_la<float, 64>; return true;
            default: return false;
        }
    }
    switch (d) {
        case 16: *out = launch_la<bf16, 16>; return true;
        case 32: *out = launch_la<bf16, 32>; return true;
        case 64: *out = launch_la<bf16, 64>; return true;
        case 128: *out = launch_la<bf16, 128>; return true;
        default: return false;
    }
}

}  // namespace hla
