// la_dispatch.hip -- instances of the chunked first-order linear-attention
// kernels (la_kernels.h) and their run-time lookup.
#include "la_kernels.h"
#include "launch.h"

namespace hla {

template <typename T, int D, bool SYM>
hipError_t launch_la(const LaParams &p, hipStream_t s, bool summaries) {
    constexpr int C = kLaChunk;
    using Cfg = LaCfg<T, D, C, SYM>;
    if (summaries && p.nseg > 1) {
        hipLaunchKernelGGL((la_summary_kernel<T, D, C, SYM>), dim3((p.nseg - 1) * p.BH),
                           dim3(Cfg::NT), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((la_forward_kernel<T, D, C, SYM>), dim3(p.nseg * p.BH), dim3(Cfg::NT), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D>
bool la_pair(LaLaunch *plain, LaLaunch *sym) {
    static_assert(sizeof(LaLds<T, D, kLaChunk, true>) <= 160 * 1024, "LDS");
    *plain = launch_la<T, D, false>;
    *sym = launch_la<T, D, true>;
    return true;
}

bool lookup_la(int dtype, int d, LaLaunch *plain, LaLaunch *sym) {
    if (dtype == 0) {
        switch (d) {
            case 16: return la_pair<float, 16>(plain, sym);
            case 32: return la_pair<float, 32>(plain, sym);
            case 64: return la_pair<float, 64>(plain, sym);
            default: return false;
        }
    }
    switch (d) {
        case 16: return la_pair<bf16, 16>(plain, sym);
        case 32: return la_pair<bf16, 32>(plain, sym);
        case 64: return la_pair<bf16, 64>(plain, sym);
        case 128: return la_pair<bf16, 128>(plain, sym);
        default: return false;
    }
}

}  // namespace hla
