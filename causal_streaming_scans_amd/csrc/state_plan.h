// state_plan.h -- which wave holds which 16x16 tiles of the carried state,
// and whether it advances them before or after the chunk's mid barrier.
//
// The chunk kernels give each wave one row tile R of the chunk.  The causal
// products of the chunk (scores, L K, tril(Q Z^T), P V) cost a wave R + 1
// tile steps, so the waves of late row tiles carry up to four times the
// triangular work of row tile 0.  The state update is the work that can be
// moved: each tile of S, W (and C) is the same product for whichever wave
// holds it.  A plan lists, per row tile, the groups of tiles that wave holds.
// Products that read only the staged chunk (S += K^T K, C += Q^T V) may run
// before the mid barrier, where the light waves otherwise wait for the heavy
// ones; products of Z (W, u) run after it.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace hla {

// Matrices of the carried state and of a segment summary, in 16x16 tiles.
// kU and kM are the column stripes u = Z^T 1 and m = Q^T 1: the products
// with a ones column tile, held as the column tile after the last one of W
// (resp. C).
enum : int { kS = 0, kW = 1, kU = 2, kC = 3, kM = 4 };

// An nr x nc rectangle of tiles of one matrix, held as the accumulators
// acc[first + nc * x + y].  ti >= 0: fixed origin (ti, tj).  ti < 0: slot
// -ti-1 of the round-robin layout, placed at run time by the wave index.
// ph: 0 = advanced before the chunk's mid barrier, 1 = after it.
struct Grp {
    int mat, ph, nr, nc, first, ti, tj;
};

template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Blocks of an (nTR x nTC)-tile matrix for NW waves: with WIDE, 2 x 4 when
// that gives every wave exactly one block (8 waves at d = 128: six operand
// reads per eight products instead of eight), else TileBlocks' square ones.
template <int nTR, int nTC, int NW, bool WIDE>
struct RectBlocks {
    using Sq = TileBlocks<nTR, nTC, NW>;
    static constexpr bool wide = WIDE && nTR % 2 == 0 && nTC % 4 == 0 && nTR * nTC == 8 * NW;
    static constexpr int BRr = wide ? 2 : Sq::BR, BRc = wide ? 4 : Sq::BR;
    static constexpr int nBR = nTR / BRr, nBC = nTC / BRc, NB = nBR * nBC;
    static constexpr int PB = (NB + NW - 1) / NW;
};

// The even layout for any shape: the blocks of S and of W (and C) dealt to
// the waves in turn, then the stripe tiles, all advanced after the barrier.
// The summary takes 2 x 4 blocks where RectBlocks gives them (d = 128
// summary 148 -> 137 us); the forward keeps square ones, since its chunk
// loop has no registers left for the wider operand sets (with them its
// spills doubled and the d = 128 forward went from 239 to 256 us).
template <int nTD, int nTV, int NW, bool SUM>
struct RoundRobinPlan {
    using SB = RectBlocks<nTD, nTD, NW, SUM>;
    using WB = RectBlocks<nTD, nTV, NW, SUM>;
    static constexpr int UJ = (nTD + NW - 1) / NW;
    static constexpr int NMW = SUM ? 2 : 1;   // W, and C in a summary
    static constexpr int aS = SB::BRr * SB::BRc, aW = WB::BRr * WB::BRc;
    static constexpr int NG = SB::PB + NMW * WB::PB + NMW * UJ;
    static constexpr int NA = SB::PB * aS + NMW * WB::PB * aW + NMW * UJ;

    static constexpr Grp grp(int i) {
        int base = 0;
        if (i < SB::PB) return Grp{kS, 1, SB::BRr, SB::BRc, i * aS, -(i + 1), 0};
        i -= SB::PB;
        base += SB::PB * aS;
        if (i < WB::PB) return Grp{kW, 1, WB::BRr, WB::BRc, base + i * aW, -(i + 1), 0};
        i -= WB::PB;
        base += WB::PB * aW;
        if (SUM) {
            if (i < WB::PB) return Grp{kC, 1, WB::BRr, WB::BRc, base + i * aW, -(i + 1), 0};
            i -= WB::PB;
            base += WB::PB * aW;
        }
        if (i < UJ) return Grp{kU, 1, 1, 1, base + i, -(i + 1), nTV};
        i -= UJ;
        base += UJ;
        return Grp{kM, 1, 1, 1, base + i, -(i + 1), nTV};
    }
    template <int I>
    __device__ static __forceinline__ bool origin(int w, int &ti, int &tj) {
        constexpr Grp g = grp(I);
        const int slot = -g.ti - 1;
        if constexpr (g.mat == kU || g.mat == kM) {
            ti = w + slot * NW;
            tj = nTV;
            return ti < nTD;
        } else {
            using TB = std::conditional_t<g.mat == kS, SB, WB>;
            const int blk = w + slot * NW;
            ti = (blk / TB::nBC) * TB::BRr;
            tj = (blk % TB::nBC) * TB::BRc;
            return blk < TB::NB;
        }
    }
};

// A plan given as a fixed table per row tile (first is filled in by the order
// of the entries).
template <typename Tab, int R>
struct FixedPlan {
    static constexpr int NG = Tab::ng(R);
    static constexpr Grp grp(int i) {
        Grp g = Tab::g(R, i);
        int first = 0;
        for (int k = 0; k < i; ++k) {
            const Grp h = Tab::g(R, k);
            first += h.nr * h.nc;
        }
        g.first = first;
        return g;
    }
    static constexpr int na() {
        int n = 0;
        for (int k = 0; k < NG; ++k) n += Tab::g(R, k).nr * Tab::g(R, k).nc;
        return n;
    }
    static constexpr int NA = na();
    template <int I>
    __device__ static __forceinline__ bool origin(int, int &ti, int &tj) {
        constexpr Grp g = grp(I);
        ti = g.ti;
        tj = g.tj;
        return true;
    }
};

// HLA-2 forward, chunk 64, d = dv = 64, one wave per row tile.  Per-wave cost
// of a chunk in 16x16x16 MFMA steps: before the mid barrier 44 + 8R (scores,
// Z, Q W0), after it 9(R + 1) (tril(Q Z^T), P V, the denominator).  S blocks
// go to the early barrier slot of waves 0-2, W and u fill the late slot
// heaviest-last: 68 before and 44-49 after, where the even layout costs the
// last wave 68 + 72.
struct Hla2Fwd64Tab {
    static constexpr int ng(int r) { return r == 0 ? 5 : r == 1 ? 4 : r == 2 ? 3 : 1; }
    static constexpr Grp g(int r, int i) {
        constexpr Grp t[4][5] = {
            {{kS, 0, 2, 2, 0, 0, 0}, {kS, 0, 1, 2, 0, 2, 2}, {kW, 1, 2, 2, 0, 0, 0}, {kW, 1, 2, 2, 0, 0, 2},
             {kS, 1, 1, 2, 0, 2, 0}},
            {{kS, 0, 2, 2, 0, 0, 2}, {kW, 1, 2, 2, 0, 2, 0}, {kS, 1, 1, 2, 0, 3, 0}, {kU, 1, 1, 1, 0, 0, 4},
             {}},
            {{kS, 0, 1, 2, 0, 3, 2}, {kW, 1, 2, 2, 0, 2, 2}, {kU, 1, 1, 1, 0, 1, 4}, {}, {}},
            {{kU, 1, 2, 1, 0, 2, 4}, {}, {}, {}, {}},
        };
        return t[r][i];
    }
};

// HLA-2 segment summary, same shape.  Before the barrier 8(R + 1) + 16
// (scores, Z); S, C and m read only the staged chunk and are dealt so that
// every wave reaches 72; after it each wave advances one W block and one u
// tile (20).  The even layout costs the last wave 48 + 56.
struct Hla2Sum64Tab {
    static constexpr int ng(int r) { return r == 0 ? 5 : r == 1 ? 5 : r == 2 ? 4 : 4; }
    static constexpr Grp g(int r, int i) {
        constexpr Grp t[4][5] = {
            {{kS, 0, 2, 2, 0, 0, 0}, {kS, 0, 2, 2, 0, 0, 2}, {kC, 0, 2, 2, 0, 0, 0}, {kW, 1, 2, 2, 0, 0, 0},
             {kU, 1, 1, 1, 0, 0, 4}},
            {{kS, 0, 2, 2, 0, 2, 0}, {kC, 0, 2, 2, 0, 0, 2}, {kM, 0, 2, 1, 0, 0, 4}, {kW, 1, 2, 2, 0, 0, 2},
             {kU, 1, 1, 1, 0, 1, 4}},
            {{kS, 0, 2, 2, 0, 2, 2}, {kC, 0, 2, 2, 0, 2, 0}, {kW, 1, 2, 2, 0, 2, 0}, {kU, 1, 1, 1, 0, 2, 4},
             {}},
            {{kC, 0, 2, 2, 0, 2, 2}, {kM, 0, 2, 1, 0, 2, 4}, {kW, 1, 2, 2, 0, 2, 2}, {kU, 1, 1, 1, 0, 3, 4},
             {}},
        };
        return t[r][i];
    }
};

// A fixed table holds every tile of the state exactly once over the RT row
// tiles (S, W, u; with C and m in a summary), and nothing else.
template <typename Tab>
constexpr bool plan_exact(int RT, int nTD, int nTV, bool sum) {
    for (int mat = kS; mat <= kM; ++mat) {
        const bool present = mat == kS || mat == kW || mat == kU || sum;
        const int c0 = (mat == kU || mat == kM) ? nTV : 0;
        const int c1 = mat == kS ? nTD : nTV + ((mat == kU || mat == kM) ? 1 : 0);
        for (int ti = 0; ti < nTD; ++ti)
            for (int tj = c0; tj < c1; ++tj) {
                int n = 0;
                for (int r = 0; r < RT; ++r)
                    for (int i = 0; i < Tab::ng(r); ++i) {
                        const Grp g = Tab::g(r, i);
                        if (g.mat == mat && ti >= g.ti && ti < g.ti + g.nr && tj >= g.tj && tj < g.tj + g.nc) ++n;
                    }
                if (n != (present ? 1 : 0)) return false;
            }
    }
    for (int r = 0; r < RT; ++r)
        for (int i = 0; i < Tab::ng(r); ++i) {
            const Grp g = Tab::g(r, i);
            const int cols = g.mat == kS ? nTD : nTV + ((g.mat == kU || g.mat == kM) ? 1 : 0);
            if (g.nr < 1 || g.nc < 1 || g.ti + g.nr > nTD || g.tj + g.nc > cols) return false;
            if (!sum && (g.mat == kC || g.mat == kM)) return false;
            if ((g.mat == kW || g.mat == kU) && g.ph != 1) return false;   // products of Z
        }
    return true;
}
static_assert(plan_exact<Hla2Fwd64Tab>(4, 4, 4, false), "forward plan covers the state once");
static_assert(plan_exact<Hla2Sum64Tab>(4, 4, 4, true), "summary plan covers the state once");

// f(gi, ti0, tj0) for every group of plan P this wave holds whose matrix is
// MAT and phase PH (-1: any); gi is the group index as a compile-time constant.
template <typename P, int MAT, int PH, typename F>
__device__ __forceinline__ void for_groups(int w, F &&f) {
    static_for<P::NG>([&](auto gi) {
        constexpr int I = decltype(gi)::value;
        constexpr Grp g = P::grp(I);
        if constexpr ((MAT < 0 || g.mat == MAT) && (PH < 0 || g.ph == PH)) {
            int ti, tj;
            if (P::template origin<I>(w, ti, tj)) f(gi, ti, tj);
        }
    });
}

// f(j, ti, tj) for every tile of matrix MAT this wave holds: j indexes the
// accumulators, (ti, tj) is the tile (tj of a stripe is its column tile).
template <typename P, int MAT, typename F>
__device__ __forceinline__ void for_tiles(int w, F &&f) {
    for_groups<P, MAT, -1>(w, [&](auto gi, int ti0, int tj0) {
        constexpr Grp g = P::grp(decltype(gi)::value);
#pragma unroll
        for (int x = 0; x < g.nr; ++x)
#pragma unroll
            for (int y = 0; y < g.nc; ++y) f(g.first + g.nc * x + y, ti0 + x, tj0 + y);
    });
}

// acc[NC x + y] += sum_k A[k][ca + 16x + i] * B[k][cb + 16y + j], k = 0..K,
// over the rows of two LdsTile matrices: an NR x NC rectangle of tiles
// sharing its operands.  ONES: B is the ones column tile instead.
template <int NR, int NC, int K, typename TA, typename TB, bool ONES>
__device__ __forceinline__ void mma_tn_grp(f32x4 *acc, const bf16 *A, int ca, const bf16 *B, int cb) {
    if constexpr (K % 32 == 0) {
#pragma unroll
        for (int k = 0; k < K; k += 32) {
            bf16x8 a[NR], b[NC];
#pragma unroll
            for (int x = 0; x < NR; ++x) a[x] = ld_op8_tt<TA>(A, k, ca + 16 * x);
#pragma unroll
            for (int y = 0; y < NC; ++y) b[y] = ONES ? ones_op8() : ld_op8_tt<TB>(B, k, cb + 16 * y);
#pragma unroll
            for (int x = 0; x < NR; ++x)
#pragma unroll
                for (int y = 0; y < NC; ++y)
                    acc[NC * x + y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[x], b[y], acc[NC * x + y], 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; k += 16) {
            Frag16<bf16> a[NR], b[NC];
#pragma unroll
            for (int x = 0; x < NR; ++x) a[x] = ld_frag_tt<TA>(A, k, ca + 16 * x);
#pragma unroll
            for (int y = 0; y < NC; ++y) b[y] = ONES ? ones_frag<bf16>() : ld_frag_tt<TB>(B, k, cb + 16 * y);
#pragma unroll
            for (int x = 0; x < NR; ++x)
#pragma unroll
                for (int y = 0; y < NC; ++y) acc[NC * x + y] = mma16(acc[NC * x + y], a[x], b[y]);
        }
    }
}
template <int NR, int NC, int K, typename TA, typename TB, bool ONES>
__device__ __forceinline__ void mma_tn_grp(f32x4 *acc, const float *A, int ca, const float *B, int cb) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll 4
    for (int k = 0; k < K; k += 4) {
        float a[NR], b[NC];
#pragma unroll
        for (int x = 0; x < NR; ++x) a[x] = A[TA::off(k + g, ca + 16 * x + r)];
#pragma unroll
        for (int y = 0; y < NC; ++y) b[y] = ONES ? (r == 0 ? 1.f : 0.f) : B[TB::off(k + g, cb + 16 * y + r)];
#pragma unroll
        for (int x = 0; x < NR; ++x)
#pragma unroll
            for (int y = 0; y < NC; ++y)
                acc[NC * x + y] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], b[y], acc[NC * x + y], 0, 0, 0);
    }
}

}  // namespace hla
