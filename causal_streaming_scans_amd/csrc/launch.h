// launch.h -- internal dispatch between the C ABI and the kernel templates.
#pragma once

#include <hip/hip_runtime.h>

#include "params.h"
#include "../../include/hla.h"

namespace hla {

typedef hipError_t (*FwdLaunch)(const FwdParams &, hipStream_t);
typedef hipError_t (*StepLaunch)(const StepParams &, hipStream_t);

struct FwdKernels {
    FwdLaunch summary;   // grid (nseg-1, BH): segment summaries from zero state
    FwdLaunch up_sweep;  // one launch per level, grid (pairs, BH): up-sweep of the scan
    FwdLaunch forward;   // grid (nseg, BH): prefix from the up-sweep nodes, chunked forward
    FwdLaunch forward_z; // the same, also writing the first pass's rows to p.z_out (HLA-2: Z, AHLA: Y)
};

// dtype: 0 = fp32, 1 = bf16.  ahla: AHLA family (else HLA-2).  Returns false
// when no instance exists for these compile-time parameters.
bool lookup_forward(int dtype, bool ahla, int d, int dv, int chunk, bool decay, FwdKernels *out);
// mode: StepMode (HLA-2, AHLA, third order)
bool lookup_step(int dtype, int mode, int d, int dv, StepLaunch *out);

// per-(dtype, d) tables, one translation unit each
bool lookup_forward_f32_16(bool ahla, int chunk, bool decay, FwdKernels *out);
bool lookup_forward_f32_32(bool ahla, int chunk, bool decay, FwdKernels *out);
bool lookup_forward_f32_64(bool ahla, int chunk, bool decay, FwdKernels *out);
bool lookup_forward_bf16_16(bool ahla, int chunk, bool decay, FwdKernels *out);
bool lookup_forward_bf16_32(bool ahla, int chunk, bool decay, FwdKernels *out);
bool lookup_forward_bf16_64(bool ahla, int chunk, bool decay, FwdKernels *out);
bool lookup_forward_bf16_128(bool ahla, int chunk, bool decay, FwdKernels *out);

// Chunked first-order linear attention (la_kernels.h): the segment-state
// launch (when p.nseg > 1 and `summaries`; otherwise p.sums must already hold
// the states of these b, c and decay) and the main launch, on one stream;
// `plain` runs LA(a, b, c), `sym` the two-slot form LA(a, b, c) + LA(a, c, b),
// `dual` LA(a, b, c) into out and LA(a2, c, b) into out2.
constexpr int kLaChunk = 64;
typedef hipError_t (*LaLaunch)(const LaParams &, hipStream_t, bool summaries);
struct LaLaunches {
    LaLaunch plain, sym, dual;
    // the segment-state launch of the plain form alone (when p.nseg > 1)
    hipError_t (*states)(const LaParams &, hipStream_t);
    // three such launches (same BH, n, segments) as one: p3[0..2]
    hipError_t (*states3)(const LaParams *p3, hipStream_t);
    hipError_t (*unit_column)(void *out, long rows, hipStream_t);   // rows (1, 0, ..., 0)
    hipError_t (*ratio_prep)(const RatioPrepParams &, hipStream_t);
    // both steps of the decay gradient; p.nblk is set by the host
    hipError_t (*decay_grad)(const DecayGradParams &, hipStream_t);
};
bool lookup_la(int dtype, int d, LaLaunches *out);
// out[t][:] = num[t][:] / den[t][0] over rows of d fp32 values; out is bf16
// (to_bf16) or fp32
hipError_t launch_divide_rows(const float *num, const float *den, void *out, long rows, int d,
                              bool to_bf16, hipStream_t s);
// bf16 -> fp32 (to_f32) or fp32 -> bf16 copy of count values (a multiple of 4)
hipError_t launch_convert(const void *src, void *dst, long count, bool to_f32, hipStream_t s);

// hla_forward's argument checks, except the workspace's, with no HIP call;
// on HLA_OK *need holds the workspace bytes the call needs (hla_api.cpp)
hla_status forward_validate(const void *q, const void *k, const void *v, void *o, int B, int H,
                            int n, int d, int dv, int dtype, int variant, const float *gamma_host,
                            int chunk, int seg_chunks, const float *state_in, float *state_out,
                            size_t *need);

// fill dst[0:count) with src[0:count), or with zeros when src is null
hipError_t launch_copy_or_zero(const float *src, float *dst, size_t count, hipStream_t s);

}  // namespace hla
