// chunk_common.h -- pieces shared by the chunk kernels of HLA-2 and AHLA.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "params.h"

namespace hla {

// Waves per workgroup for a chunk of C tokens and head size D: one row tile of
// 16 tokens per wave group, column groups added until there are 4 waves (8 for
// D >= 128, whose fp32 state needs the registers of 8 waves).
template <int C, int D>
struct WaveShape {
    static constexpr int RT = C / 16;                       // row tiles per chunk
    static constexpr int target = D >= 128 ? 8 : 4;
    static constexpr int ncg0 = target / RT > 0 ? target / RT : 1;
    static constexpr int NCG = ncg0 < D / 16 ? ncg0 : D / 16;  // column groups
    static constexpr int NW = RT * NCG;
    static constexpr int NT = NW * kWave;
};

// f(std::integral_constant<int, r>) for the wave-uniform row tile r in
// [0, RT): each wave runs the intra-chunk phases unrolled for its own row
// tile, with no per-tile branches, so every operand load of a phase can be
// issued ahead of its products.
template <int RT, int I = 0, typename F>
__device__ __forceinline__ void with_row_tile(int r, F &&f) {
    if constexpr (I < RT) {
        if (r == I) f(std::integral_constant<int, I>{});
        else with_row_tile<RT, I + 1>(r, static_cast<F &&>(f));
    }
}

// One thread's share of a [C][COLS] chunk tile, held in registers between the
// global load (issued a chunk ahead) and the LDS store.  The loads are
// unconditional -- a row past the end of the sequence reads row 0 of the
// chunk instead (always in bounds) -- and the raw 16-byte values are kept
// whole; rows past the end are zeroed only when stored to LDS.  So nothing
// consumes a load until the next chunk is staged, and no wait for it lands
// in the middle of the current chunk.
//
// Lanes run along the columns of a row (item idx -> row idx / VPR, 16-byte
// column group idx % VPR): one load instruction covers whole rows, i.e.
// whole cache lines, and the row-major LDS store writes whole rows.  With
// lanes along the tokens instead, every lane of a load touches its own cache
// line and the vector memory path handles eight times the line requests.
template <typename T, int C, int COLS, int NT>
struct ChunkRegs {
    static constexpr int VE = Vec16<T>::N;
    static constexpr int VPR = COLS / VE;
    static constexpr int NVEC = C * VPR;
    static constexpr int NV = (NVEC + NT - 1) / NT;
    static_assert(COLS % VE == 0, "rows of whole 16-byte groups");
    uint4 raw[NV];

    // rows at or past rv read as zeros: the loads go through a buffer
    // resource that covers the rv valid rows only, whose range check returns
    // zeros past its end, so neither the loads nor the staging stores need a
    // per-row select (each 16-byte piece lies wholly inside or outside)
    __device__ __forceinline__ void load(const T *__restrict__ src, int rv) {
        const __amdgpu_buffer_rsrc_t rs = rows_rsrc(src, rv, COLS);
#pragma unroll
        for (int i = 0; i < NV; ++i) raw[i] = load16_buf(rs, (threadIdx.x + i * NT) * 16);
    }
    __device__ __forceinline__ Vec16<T> get(int i) const {
        Vec16<T> x;
        *reinterpret_cast<uint4 *>(x.v) = raw[i];
        return x;
    }
    // the same into an LdsTile matrix
    template <typename TL>
    __device__ __forceinline__ void store_tile(T *dst) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + i * NT;
            if (idx < NVEC) store16(dst + TL::off(idx / VPR, (idx % VPR) * VE), get(i));
        }
    }
    template <typename TL>
    __device__ __forceinline__ void store_tile_w(T *dst, const float *gp, int wofs) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + i * NT;
            if (idx < NVEC) {
                const int r = idx / VPR;
                const float wr = r <= wofs ? gp[wofs - r] : 0.f;
                Vec16<T> x = get(i);
#pragma unroll
                for (int e = 0; e < VE; ++e) x.v[e] = from_f<T>(to_f(x.v[e]) * wr);
                store16(dst + TL::off(r, (idx % VPR) * VE), x);
            }
        }
    }
};




}  // namespace hla
