// la_dispatch.hip -- instances of the chunked first-order linear-attention
// kernels (la_kernels.h) and their run-time lookup.
#include "la_kernels.h"
#include "launch.h"

namespace hla {

// Chunk of the kernels: 64 tokens, or 32 for fp32 at d >= 32, whose 64-token
// tiles would leave room for one workgroup per compute unit.  Segments are
// multiples of kLaChunk tokens either way.
template <typename T, int D>
constexpr int la_chunk() { return (sizeof(T) == 4 && D >= 32) ? 32 : kLaChunk; }

template <typename T, int D, bool SYM, bool DUAL>
hipError_t launch_la(const LaParams &p, hipStream_t s, bool summaries) {
    constexpr int C = la_chunk<T, D>();
    using Cfg = LaCfg<T, D, C, SYM, DUAL>;
    if (summaries && p.nseg > 1) {
        // a DUAL pass's state is the plain state of its b, c
        hipLaunchKernelGGL((la_summary_kernel<T, D, C, SYM, false>), dim3((p.nseg - 1) * p.BH),
                           dim3(Cfg::NT), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((la_forward_kernel<T, D, C, SYM, DUAL>), dim3(p.nseg * p.BH), dim3(Cfg::NT),
                       0, s, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_la_states(const LaParams &p, hipStream_t s) {
    constexpr int C = la_chunk<T, D>();
    if (p.nseg <= 1) return hipSuccess;
    hipLaunchKernelGGL((la_summary_kernel<T, D, C, false, false>), dim3((p.nseg - 1) * p.BH),
                       dim3(LaCfg<T, D, C, false, false>::NT), 0, s, p);
    return hipGetLastError();
}

// the segment states of three plain passes with the same sizes (nseg > 1)
template <typename T, int D>
hipError_t launch_la_states3(const LaParams *p3, hipStream_t s) {
    constexpr int C = la_chunk<T, D>();
    if (p3[0].nseg <= 1) return hipSuccess;
    LaParams3 ps;
    for (int i = 0; i < 3; ++i) ps.p[i] = p3[i];
    hipLaunchKernelGGL((la_summary3_kernel<T, D, C>), dim3(3 * (p3[0].nseg - 1) * p3[0].BH),
                       dim3(LaCfg<T, D, C, false, false>::NT), 0, s, ps);
    return hipGetLastError();
}

// The DUAL form as two plain passes, for shapes whose fused LDS layout does
// not fit: LA(a, b, c) into out, then LA(a2, c, b) into out2.
template <typename T, int D>
hipError_t launch_la_dual_split(const LaParams &p, hipStream_t s, bool summaries) {
    hipError_t e = launch_la<T, D, false, false>(p, s, summaries);
    if (e != hipSuccess) return e;
    LaParams q = p;
    q.a = p.a2;
    q.b = p.c;
    q.c = p.b;
    q.add = p.add2;
    q.out = p.out2;
    q.a2 = nullptr;
    q.out2 = nullptr;
    q.add2 = nullptr;
    return launch_la<T, D, false, false>(q, s, true);
}

// The SYM form as two plain passes, for shapes whose fused LDS layout does
// not fit: LA(a, b, c) into out (after add), then LA(a, c, b) added to it.
template <typename T, int D>
hipError_t launch_la_sym_split(const LaParams &p, hipStream_t s, bool summaries) {
    hipError_t e = launch_la<T, D, false, false>(p, s, summaries);
    if (e != hipSuccess) return e;
    LaParams q = p;
    q.b = p.c;
    q.c = p.b;
    q.add = p.out;
    return launch_la<T, D, false, false>(q, s, true);
}

template <typename T, int D>
hipError_t launch_unit_column(void *out, long rows, hipStream_t s) {
    long blocks = (rows * D + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL((unit_column_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<T *>(out), rows);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_ratio_prep(const RatioPrepParams &p, hipStream_t s) {
    const long blocks = (p.rows + 3) / 4;   // one wave per row, four waves per block
    hipLaunchKernelGGL((ratio_prep_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decay_grad(const DecayGradParams &p, hipStream_t s) {
    // nblk == 0 (no rows): the second step alone writes zeros
    if (p.nblk < 0 || p.nblk > kDecayGradBlocks || p.BH < 1 || p.H < 1 || p.BH % p.H != 0)
        return hipErrorInvalidValue;
    if (p.nblk > 0) {
        hipLaunchKernelGGL((decay_grad_rows_kernel<T, D>), dim3((unsigned)p.nblk, (unsigned)p.BH),
                           dim3(256), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(decay_grad_final_kernel, dim3((unsigned)p.H), dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D>
bool la_set(LaLaunches *out) {
    out->unit_column = launch_unit_column<T, D>;
    out->ratio_prep = launch_ratio_prep<T, D>;
    out->decay_grad = launch_decay_grad<T, D>;
    static_assert(sizeof(LaLds<T, D, la_chunk<T, D>(), false, false>) <= 160 * 1024, "LDS");
    out->plain = launch_la<T, D, false, false>;
    out->states = launch_la_states<T, D>;
    out->states3 = launch_la_states3<T, D>;
    if constexpr (sizeof(LaLds<T, D, la_chunk<T, D>(), true, false>) <= 160 * 1024)
        out->sym = launch_la<T, D, true, false>;
    else
        out->sym = launch_la_sym_split<T, D>;
    if constexpr (sizeof(LaLds<T, D, la_chunk<T, D>(), false, true>) <= 160 * 1024)
        out->dual = launch_la<T, D, false, true>;
    else
        out->dual = launch_la_dual_split<T, D>;
    return true;
}

template <int D>
hipError_t launch_divide_rows_d(const float *num, const float *den, void *out, long rows,
                                bool to_bf16, hipStream_t s) {
    long blocks = (rows * (D / 4) + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) return hipSuccess;
    if (to_bf16)
        hipLaunchKernelGGL((divide_rows_kernel<bf16, D>), dim3((unsigned)blocks), dim3(256), 0, s,
                           num, den, static_cast<bf16 *>(out), rows);
    else
        hipLaunchKernelGGL((divide_rows_kernel<float, D>), dim3((unsigned)blocks), dim3(256), 0, s,
                           num, den, static_cast<float *>(out), rows);
    return hipGetLastError();
}

hipError_t launch_divide_rows(const float *num, const float *den, void *out, long rows, int d,
                              bool to_bf16, hipStream_t s) {
    switch (d) {
        case 16: return launch_divide_rows_d<16>(num, den, out, rows, to_bf16, s);
        case 32: return launch_divide_rows_d<32>(num, den, out, rows, to_bf16, s);
        case 64: return launch_divide_rows_d<64>(num, den, out, rows, to_bf16, s);
        case 128: return launch_divide_rows_d<128>(num, den, out, rows, to_bf16, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_convert(const void *src, void *dst, long count, bool to_f32, hipStream_t s) {
    const long count4 = count / 4;
    long blocks = (count4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) return hipSuccess;
    if (to_f32)
        hipLaunchKernelGGL(widen_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const bf16 *>(src), static_cast<float *>(dst), count4);
    else
        hipLaunchKernelGGL(narrow_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const float *>(src), static_cast<bf16 *>(dst), count4);
    return hipGetLastError();
}

bool lookup_la(int dtype, int d, LaLaunches *out) {
    if (dtype == 0) {
        switch (d) {
            case 16: return la_set<float, 16>(out);
            case 32: return la_set<float, 32>(out);
            case 64: return la_set<float, 64>(out);
            case 128: return la_set<float, 128>(out);
            default: return false;
        }
    }
    switch (d) {
        case 16: return la_set<bf16, 16>(out);
        case 32: return la_set<bf16, 32>(out);
        case 64: return la_set<bf16, 64>(out);
        case 128: return la_set<bf16, 128>(out);
        default: return false;
    }
}

}  // namespace hla
