// dispatch.hip -- decode-step instances, the small copy kernel, and the
// run-time lookup from argument values to kernel instances.
#include "launch.h"
#include "step_kernel.h"

namespace hla {

__global__ void copy_or_zero_kernel(const float *src, float *dst, size_t count) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_or_zero(const float *src, float *dst, size_t count, hipStream_t s) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, count);
    return hipGetLastError();
}

template <typename T, int D, int MODE>
hipError_t launch_step(const StepParams &p, hipStream_t s) {
    if constexpr (MODE == kStepHla3) {
        hipLaunchKernelGGL((hla3_step_kernel<T, D, D, 256>), dim3(p.BH), dim3(256), 0, s, p);
    } else if (MODE == kStepAhla && !p.ratio) {
        // unnormalised AHLA: one workgroup per 16 value columns of each head
        hipLaunchKernelGGL((ahla_step_sliced_kernel<T, D, D, 256>), dim3(p.BH * (D / 16)), dim3(256),
                           0, s, p);
    } else {
        hipLaunchKernelGGL((step_kernel<T, D, D, MODE, 256>), dim3(p.BH), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

template <typename T, int D>
static StepLaunch step_mode(int mode) {
    return mode == kStepAhla ? launch_step<T, D, kStepAhla>
         : mode == kStepHla3 ? launch_step<T, D, kStepHla3> : launch_step<T, D, kStepHla2>;
}

template <typename T>
static bool step_for(int mode, int d, StepLaunch *out) {
    switch (d) {
        case 16: *out = step_mode<T, 16>(mode); return true;
        case 32: *out = step_mode<T, 32>(mode); return true;
        case 64: *out = step_mode<T, 64>(mode); return true;
        case 128: *out = step_mode<T, 128>(mode); return true;
        default: return false;
    }
}

bool lookup_step(int dtype, int mode, int d, int dv, StepLaunch *out) {
    if (d != dv) return false;
    return dtype == 0 ? step_for<float>(mode, d, out) : step_for<bf16>(mode, d, out);
}

bool lookup_forward(int dtype, bool ahla, int d, int dv, int chunk, bool decay, FwdKernels *out) {
    if (d != dv) return false;
    if (dtype == 0) {
        switch (d) {
            case 16: return lookup_forward_f32_16(ahla, chunk, decay, out);
            case 32: return lookup_forward_f32_32(ahla, chunk, decay, out);
            case 64: return lookup_forward_f32_64(ahla, chunk, decay, out);
            default: return false;
        }
    }
    switch (d) {
        case 16: return lookup_forward_bf16_16(ahla, chunk, decay, out);
        case 32: return lookup_forward_bf16_32(ahla, chunk, decay, out);
        case 64: return lookup_forward_bf16_64(ahla, chunk, decay, out);
        case 128: return lookup_forward_bf16_128(ahla, chunk, decay, out);
        default: return false;
    }
}

}  // namespace hla
