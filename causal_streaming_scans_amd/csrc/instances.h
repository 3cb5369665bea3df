// instances.h -- kernel instantiation for one (element type, head dim); each
// inst_*.hip includes this once so the instances compile in parallel.
#pragma once

#include "ahla_kernels.h"
#include "hla2_kernels.h"
#include "hla2_pipe.h"
#include "launch.h"

namespace hla {

constexpr size_t kLdsBytes = 160 * 1024;   // gfx950 LDS per workgroup

template <typename T, int D, int C, bool DECAY>
constexpr bool hla2_fits() {
    return sizeof(Hla2FwdLds<T, D, D, C, DECAY>) <= kLdsBytes &&
           sizeof(Hla2SumSmem<T, D, D, C, DECAY>) <= kLdsBytes;
}

template <typename T, int D, int C, bool DECAY>
constexpr bool ahla_fits() {
    return sizeof(AhlaFwdLds<T, D, D, C, DECAY>) <= kLdsBytes &&
           sizeof(AhlaSumSmem<T, D, D, C, DECAY>) <= kLdsBytes;
}

template <typename T, int D, int C, bool DECAY>
hipError_t launch_hla2_summary(const FwdParams &p, hipStream_t s) {
    hipLaunchKernelGGL((hla2_summary_kernel<T, D, D, C, DECAY>), dim3(p.nseg - 1, p.BH),
                       dim3(Hla2Cfg<T, D, D, C, DECAY>::NT), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D, int C, bool DECAY, bool ZO = false>
hipError_t launch_hla2_forward(const FwdParams &p, hipStream_t s) {
    hipLaunchKernelGGL((hla2_forward_kernel<T, D, D, C, DECAY, ZO>), dim3(p.nseg * p.BH),
                       dim3(Hla2Cfg<T, D, D, C, DECAY>::NT), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D, int C, bool ZO = false>
hipError_t launch_hla2_forward_pipe(const FwdParams &p, hipStream_t s) {
    hipLaunchKernelGGL((hla2_forward_pipe_kernel<T, D, D, C, ZO>), dim3(p.nseg * p.BH),
                       dim3(Hla2Cfg<T, D, D, C, false>::NT), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D, int C, bool DECAY>
hipError_t launch_ahla_summary(const FwdParams &p, hipStream_t s) {
    hipLaunchKernelGGL((ahla_summary_kernel<T, D, D, C, DECAY>), dim3(p.nseg - 1, p.BH),
                       dim3(AhlaCfg<T, D, D, C>::NT), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D, int C, bool DECAY, bool YO = false>
hipError_t launch_ahla_forward(const FwdParams &p, hipStream_t s) {
    hipLaunchKernelGGL((ahla_forward_kernel<T, D, D, C, DECAY, YO>), dim3(p.nseg * p.BH),
                       dim3(AhlaCfg<T, D, D, C>::NT), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D, bool HLA2>
hipError_t launch_up_sweep(const FwdParams &p, hipStream_t s) {
    constexpr int NT = combine_threads<D>(), CS = combine_slices<D>();
    for (int b = 0; (p.nreal >> (b + 1)) > 0; ++b) {
        const int npair = p.nreal >> (b + 1);
        hipLaunchKernelGGL((up_sweep_kernel<HLA2, D, D, NT>), dim3(up_sweep_groups<CS>(npair * p.BH)),
                           dim3(NT), 0, s, p, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int D, int C>
bool lookup_chunk(bool ahla, bool decay, FwdKernels *out) {
    if (ahla) {
        if (decay) {
            if constexpr (ahla_fits<T, D, C, true>()) {
                *out = {launch_ahla_summary<T, D, C, true>, launch_up_sweep<T, D, false>,
                        launch_ahla_forward<T, D, C, true>, launch_ahla_forward<T, D, C, true, true>};
                return true;
            }
            return false;
        }
        if constexpr (ahla_fits<T, D, C, false>()) {
            *out = {launch_ahla_summary<T, D, C, false>, launch_up_sweep<T, D, false>,
                    launch_ahla_forward<T, D, C, false>, launch_ahla_forward<T, D, C, false, true>};
            return true;
        }
        return false;
    }
    if (decay) {
        if constexpr (hla2_fits<T, D, C, true>()) {
            *out = {launch_hla2_summary<T, D, C, true>, launch_up_sweep<T, D, true>,
                    launch_hla2_forward<T, D, C, true>, launch_hla2_forward<T, D, C, true, true>};
            return true;
        }
        return false;
    }
    if constexpr (hla2_fits<T, D, C, false>()) {
        if constexpr (hla2_pipe_ok<T, D, D, C>())
            *out = {launch_hla2_summary<T, D, C, false>, launch_up_sweep<T, D, true>,
                    launch_hla2_forward_pipe<T, D, C>, launch_hla2_forward_pipe<T, D, C, true>};
        else
            *out = {launch_hla2_summary<T, D, C, false>, launch_up_sweep<T, D, true>,
                    launch_hla2_forward<T, D, C, false>, launch_hla2_forward<T, D, C, false, true>};
        return true;
    }
    return false;
}

template <typename T, int D>
bool lookup_dim(bool ahla, int chunk, bool decay, FwdKernels *out) {
    switch (chunk) {
        case 16: return lookup_chunk<T, D, 16>(ahla, decay, out);
        case 32: return lookup_chunk<T, D, 32>(ahla, decay, out);
        case 64: return lookup_chunk<T, D, 64>(ahla, decay, out);
        default: return false;
    }
}

}  // namespace hla

#define HLA_DEFINE_LOOKUP(NAME, T, D)                                                   \
    namespace hla {                                                                     \
    bool NAME(bool ahla, int chunk, bool decay, FwdKernels *out) {                      \
        return lookup_dim<T, D>(ahla, chunk, decay, out);                               \
    }                                                                                   \
    }
