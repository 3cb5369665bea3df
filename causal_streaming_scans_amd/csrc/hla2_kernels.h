// hla2_kernels.h -- chunked second-order HLA on gfx950: the segment-summary
// kernel and the forward kernel (intra-chunk products + carried state).
//
// Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
// gist.science/es/paper/2510.27258.  Section "1. HLA de Segundo Orden" gives
// the prefix moments (S^K, C^QV, m^Q), the cross-summaries (G, h) and the
// output q^T (S^K C^QV - G); section "4. ... Escaneos Asociativos" gives the
// blockwise evaluation from segment summaries.
//
// Chunk form used here (derived from those summaries; g = per-head decay):
// the key read-out z_t = S^K_t q_t turns the operator into two chained causal
// linear attentions, o_t = q_t^T W_t with W_t = g^2 W_{t-1} + z_t v_t^T
// (W = S^K C^QV - G).  For a chunk of c tokens with carried (S0, W0, u0) and
// in-chunk positions tau:
//     L   = D_g * tril(Q K^T)                         (scores, diagonal kept)
//     Z   = diag(g^(tau+1)) Q S0 + L K                rows z_t
//     P   = D_{g^2} * tril(Q Z^T)
//     O   = diag(g^(2(tau+1))) Q W0 + P V              numerator
//     den = diag(g^(2(tau+1))) Q u0 + P 1              ratio form only
//     S0 <- g^c S0 + K^T diag(g^(c-1-tau)) K
//     W0 <- g^(2c) W0 + Z^T diag(g^(2(c-1-tau))) V ,   u0 likewise with 1
// The summary kernel runs the same recurrence from a zero state over one
// segment and also accumulates C = sum g^(e-t) q v^T and m = sum g^(e-t) q,
// which the segment combine needs for its cross term.
//
// Work split.  Wave (r, cg) owns row tile r (16 tokens) of the chunk and the
// output column tiles cg, cg + NCG, ...  The scores are formed transposed
// (L^T = K Q^T), so the accumulator is directly the operand of K^T L^T (for
// Z^T) without an LDS round trip; likewise P^T = Z Q^T feeds V^T P^T (for
// O^T).  O^T's accumulator holds four consecutive output features of one
// token, so the output is written straight from registers.
//
// LDS holds chunk tiles row-major only ([token][feature]).  Every product
// that contracts over the tokens (K^T L^T, V^T P^T, the state updates) reads
// its operands with the transposing LDS read, so no transposed copy is ever
// written.  The forward kernel's Q never enters LDS: each wave reads its own
// 16 query rows from global memory into operand registers, a chunk ahead.
// A ones column tile (1, 0, ..., 0 in every row) is a constant operand
// fragment in registers: its products with Z^T, Q^T and P^T give u = Z^T 1
// (the column tile after W), m = Q^T 1 (after C) and the ratio denominator's
// P 1.  The fp32 state S0, W0 (and u0) is spread over the waves as MFMA
// accumulators for the whole segment; its T-typed transposed copy in LDS is
// the operand of Q S0 and Q W0.  Z goes through LDS, since every row tile
// needs all earlier rows of it.  Chunk tiles and state copies use the LdsTile
// layout (swizzled 128-byte rows for bf16 with 64 columns).
#pragma once

#include "chunk_common.h"
#include "combine.h"
#include "state_plan.h"

namespace hla {

template <typename T, int D, int DV, int C, bool DECAY>
struct Hla2Cfg {
    using WS = WaveShape<C, D>;
    static constexpr int RT = WS::RT, NCG = WS::NCG, NW = WS::NW, NT = WS::NT;
    static constexpr int DVX = DV + 16;       // W widened by the u column tile
    using TK = LdsTile<T, D>;                 // chunk rows of length D: Q, K, Z (and weighted copies)
    using TV = LdsTile<T, DV>;                // chunk rows of V
    using TS = LdsTile<T, D>;                 // the state copies St, Wt
    static constexpr int nTD = D / 16, nTV = DV / 16;
    static constexpr int ZJ = (nTD + NCG - 1) / NCG;    // Z^T tiles per wave
    static constexpr int OJ = (nTV + NCG - 1) / NCG;    // O^T tiles per wave
    static constexpr int UJ = (nTD + NW - 1) / NW;      // tiles of the u (m) column per wave
    using SB = TileBlocks<nTD, nTD, NW>;    // even ownership of S tiles
    using WB = TileBlocks<nTD, nTV, NW>;    // even ownership of W (and C) tiles
    // which wave holds which state tiles: a balanced table for the common
    // shape, the even round-robin layout otherwise
    static constexpr bool BAL = C == 64 && D == 64 && DV == 64 && NCG == 1;
    template <int R>
    using FwdPlan = std::conditional_t<BAL, FixedPlan<Hla2Fwd64Tab, R>, RoundRobinPlan<nTD, nTV, NW, false>>;
    template <int R>
    using SumPlan = std::conditional_t<BAL, FixedPlan<Hla2Sum64Tab, R>, RoundRobinPlan<nTD, nTV, NW, true>>;
    static constexpr int SUMF = summary_floats(D, DV);
    static constexpr int STF = hla2_state_floats(D, DV);
    static constexpr int NPOW = 2 * C + 2;
    // Output rows staged in LDS and stored whole (bf16, where the LDS has
    // room for the staging rows): wave (r, cg) holds the contiguous column
    // tiles cg*OJ .. cg*OJ+OJ-1 of its row tile, a [16][DV/NCG] tile TO.
    static constexpr bool ROWS_OUT_SHAPE = sizeof(T) == 2 && OJ * NCG == nTV;
    using TO = LdsTile<T, (ROWS_OUT_SHAPE ? DV / NCG : 16)>;
    static_assert(D % 16 == 0 && DV % 16 == 0 && C % 16 == 0, "tile multiples");
};

// Visit the tiles a wave owns in a blocked layout: f(p, x, y, ti, tj) with
// compile-time p, x, y (the accumulator indices) and run-time tile indices.
template <typename TB, int NW, typename F>
__device__ __forceinline__ void for_owned(int w, F f) {
#pragma unroll
    for (int pb = 0; pb < TB::PB; ++pb) {
        const int blk = w + pb * NW;
        if (blk < TB::NB) {
            const int bi = blk / TB::nBC, bj = blk % TB::nBC;
#pragma unroll
            for (int x = 0; x < TB::BR; ++x)
#pragma unroll
                for (int y = 0; y < TB::BR; ++y) f(pb, x, y, bi * TB::BR + x, bj * TB::BR + y);
        }
    }
}
// The blocks a wave owns: g(p, ti0, tj0) with the block's first tile.
template <typename TB, int NW, typename F>
__device__ __forceinline__ void for_blocks(int w, F f) {
#pragma unroll
    for (int pb = 0; pb < TB::PB; ++pb) {
        const int blk = w + pb * NW;
        if (blk < TB::NB) f(pb, (blk / TB::nBC) * TB::BR, (blk % TB::nBC) * TB::BR);
    }
}
// The row tiles ti of a single 16-column stripe a wave owns: f(j, ti).
template <int UJ, int NW, int NTILE, typename F>
__device__ __forceinline__ void for_stripe(int w, F f) {
#pragma unroll
    for (int j = 0; j < UJ; ++j) {
        const int ti = w + j * NW;
        if (ti < NTILE) f(j, ti);
    }
}


template <typename T, int D, int DV, int C, bool DECAY, bool RO = false>
struct Hla2FwdSmem {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    alignas(16) T K[C * G::TK::LD];
    alignas(16) T Kw[DECAY ? C * G::TK::LD : 8];    // rows weighted by g^(c-1-tau)
    alignas(16) T V[C * G::TV::LD];
    alignas(16) T Z[C * G::TK::LD];
    alignas(16) T Zw[DECAY ? C * G::TK::LD : 8];    // rows weighted by g^(2(c-1-tau))
    alignas(16) T St[D * G::TS::LD];             // St[j][i] = S0[i][j]
    alignas(16) T Wt[G::DVX * G::TS::LD];        // Wt[j][i] = W0[i][j]; row DV = u0
    alignas(16) T Ot[RO ? G::NW * 16 * G::TO::LD : 8];   // output rows on their way out
    float gp[G::NPOW];
};

// The prefix fold's cross terms on bf16 MFMA (bf16 kernels, d >= 64).  Each
// fp32 factor is split into a bf16 high part and a bf16 low part, x = h + l
// with |x - h - l| <= 2^-17 |x|, and S Y is formed as Sh Yh + Sh Yl + Sl Yh:
// the dropped Sl Yl and the rounding of the low parts leave about 2^-16 of
// each product, far inside the bf16 path's bar, and three bf16 MFMA steps
// replace eight fp32 steps per 32 k-values (with fp32 MFMA the fold cost the
// d = 128 decay forward 39 us of 250).  The old S is staged transposed (the
// layout of St) and the node's [a Y | a y | 0] row-major, each as a high and
// a low copy; fp32 kernels keep exact fp32 products for their tighter bar.
template <typename T, int D, int DV>
struct FoldX3 {
    static constexpr bool ON = sizeof(T) == 2 && D >= 64;
    using TS = LdsTile<bf16, D>;
    using TY = LdsTile<bf16, DV + 16>;
    static constexpr int S_EL = D * TS::LD, Y_EL = D * TY::LD;   // bf16 elements of one copy
    static constexpr int FLOATS = (2 * S_EL + 2 * Y_EL + 1) / 2;
};
// floats of the fold's staging area, overlaid on the chunk buffers
template <typename T, int D, int DV>
constexpr int fold_scratch_floats() {
    using X = FoldX3<T, D, DV>;
    return X::ON && X::FLOATS > CrossLds<D, DV>::FLOATS ? X::FLOATS : CrossLds<D, DV>::FLOATS;
}

// x minus its bf16 rounding (exact in fp32)
__device__ __forceinline__ f32x4 bf16_low(f32x4 x) {
    f32x4 l;
#pragma unroll
    for (int i = 0; i < 4; ++i) l[i] = x[i] - static_cast<float>(static_cast<bf16>(x[i]));
    return l;
}

// [a Y | a y | 0] of a node (fp32 rows Y [D][DV], column y [D]) into the
// high and low [D][DV+16] copies, by all NT threads
template <int D, int DV, int NT>
__device__ __forceinline__ void fold_x3_stage_y(bf16 *Yh, bf16 *Yl, const float *Y, const float *y,
                                                float a) {
    using TY = LdsTile<bf16, DV + 16>;
    constexpr int Q4 = (DV + 16) / 4, N = D * Q4;
    for (int idx = threadIdx.x; idx < N; idx += NT) {
        const int k = idx / Q4, v = 4 * (idx - k * Q4);
        f32x4 x = zero4();
        if (v < DV) x = a * *reinterpret_cast<const f32x4 *>(Y + k * DV + v);
        else if (v == DV) x[0] = a * y[k];
        store4(Yh + TY::off(k, v), x);
        store4(Yl + TY::off(k, v), bf16_low(x));
    }
}

// this wave's tiles of the old S into the high and low copies of S^T
template <typename P, int D>
__device__ __forceinline__ void fold_x3_stage_s(const f32x4 *acc, int w, bf16 *Sh, bf16 *Sl) {
    using TS = LdsTile<bf16, D>;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
        store4(Sh + TS::off(16 * tj + col, 16 * ti + g4), acc[j]);
        store4(Sl + TS::off(16 * tj + col, 16 * ti + g4), bf16_low(acc[j]));
    });
}

// W += (a S) Y, u += S (a y) for this wave's W and u groups, from the staged
// copies (the factor a travels in the staged Y)
template <typename P, int D, int DV>
__device__ __forceinline__ void fold_x3_products(f32x4 *acc, int w, const bf16 *Sh, const bf16 *Sl,
                                                 const bf16 *Yh, const bf16 *Yl) {
    using TS = LdsTile<bf16, D>;
    using TY = LdsTile<bf16, DV + 16>;
    for_groups<P, -1, -1>(w, [&](auto gi, int ti0, int tj0) {
        constexpr Grp gr = P::grp(decltype(gi)::value);
        if constexpr (gr.mat == kW || gr.mat == kU) {
            f32x4 *c = acc + gr.first;
            mma_tn_grp<gr.nr, gr.nc, D, TS, TY, false>(c, Sl, 16 * ti0, Yh, 16 * tj0);
            mma_tn_grp<gr.nr, gr.nc, D, TS, TY, false>(c, Sh, 16 * ti0, Yl, 16 * tj0);
            mma_tn_grp<gr.nr, gr.nc, D, TS, TY, false>(c, Sh, 16 * ti0, Yh, 16 * tj0);
        }
    });
}

// whether the forward stages its output rows (the shape allows it and the
// LDS holds the staging rows as well)
template <typename T, int D, int DV, int C, bool DECAY>
constexpr bool hla2_rows_out() {
    return Hla2Cfg<T, D, DV, C, DECAY>::ROWS_OUT_SHAPE &&
           sizeof(LdsWithScratch<Hla2FwdSmem<T, D, DV, C, DECAY, true>, fold_scratch_floats<T, D, DV>()>) <=
               160 * 1024;
}

template <typename T, int D, int DV, int C, bool DECAY>
using Hla2FwdLds = LdsWithScratch<Hla2FwdSmem<T, D, DV, C, DECAY, hla2_rows_out<T, D, DV, C, DECAY>()>,
                                  fold_scratch_floats<T, D, DV>()>;

template <typename T, int D, int DV, int C, bool DECAY>
struct Hla2SumSmem {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    alignas(16) T Q[C * G::TK::LD];
    alignas(16) T Qw[DECAY ? C * G::TK::LD : 8];    // rows weighted by g^(c-1-tau)
    alignas(16) T K[C * G::TK::LD];
    alignas(16) T Kw[DECAY ? C * G::TK::LD : 8];
    alignas(16) T V[C * G::TV::LD];
    alignas(16) T Z[C * G::TK::LD];                 // rows weighted by g^(2(c-1-tau))
    alignas(16) T St[D * G::TS::LD];
    float gp[G::NPOW];
};

// Workgroups per CU the kernel is built for: as many as the LDS allows, up
// to 3 (12 waves of 256-thread groups, 168 VGPRs each).
template <int NT, int SMEM>
constexpr int hla_min_blocks() {
    const int by_lds = (160 * 1024) / SMEM;
    const int cap = NT <= 256 ? 3 : 1;
    return by_lds < 1 ? 1 : (by_lds < cap ? by_lds : cap);
}
template <typename T, int D, int DV, int C, bool DECAY>
constexpr int hla2_fwd_blocks() {
    const int b = hla_min_blocks<Hla2Cfg<T, D, DV, C, DECAY>::NT, (int)sizeof(Hla2FwdLds<T, D, DV, C, DECAY>)>();
    return b > 2 ? 2 : b;
}
// The balanced plan's row tile 0 holds 17 state tiles: built for two
// workgroups per CU (the summary stage has fewer workgroups than the forward
// stage, so a third slot per CU mostly stays empty).
template <typename T, int D, int DV, int C, bool DECAY>
constexpr int hla2_sum_blocks() {
    const int b = hla_min_blocks<Hla2Cfg<T, D, DV, C, DECAY>::NT, (int)sizeof(Hla2SumSmem<T, D, DV, C, DECAY>)>();
    return Hla2Cfg<T, D, DV, C, DECAY>::BAL && b > 2 ? 2 : b;
}

// L^T tiles of row tile R as operand fragments: Lf[s] holds
// (D_g * tril(Q K^T))^T[sigma in tile s][tau in tile R], s <= R.  Only the
// diagonal tile s == R needs the causal mask.
template <typename T, int D, int R, typename TL, bool DECAY>
__device__ __forceinline__ void scores_t(Frag16<T> (&Lf)[R + 1], const T *K, const RowFrags<T, D> &qf,
                                         int tau, const float *gp, int gexp) {
    const int g4 = (lane_id() >> 4) << 2;
    f32x4 a[R + 1];
#pragma unroll
    for (int s = 0; s <= R; ++s) a[s] = mma_nt_ft<TL>(zero4(), K + 16 * s * TL::LD, qf);
#pragma unroll
    for (int s = 0; s <= R; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sigma = 16 * s + g4 + i;
            float m = a[s][i];
            if (s == R && sigma > tau) m = 0.f;
            else if (DECAY) m *= gp[gexp * (tau - sigma)];
            a[s][i] = m;
        }
        Lf[s] = to_frag<T>(a[s]);
    }
}

// Z^T tiles of row tile R: Z = diag(g^(tau+1)) Q S0 + L K, stored row-major
// (times w) into Zd.  Shared by the forward and summary kernels.
template <typename T, int D, int R, int NCG, int ZJ, typename TK, bool DECAY, typename TS>
__device__ __forceinline__ void z_tiles(const RowFrags<T, D> &qf, const Frag16<T> (&Lf)[R + 1],
                                        const T *St, const T *K, T *Zd, T *Zwd, float wz,
                                        const float *gp, int cg, int tau) {
    const int g4 = (lane_id() >> 4) << 2;
    f32x4 z[ZJ];
#pragma unroll
    for (int jj = 0; jj < ZJ; ++jj) {
        const int jt = cg + jj * NCG;
        z[jj] = zero4();
        if (jt < D / 16) {
            f32x4 zq = mma_nt_ft<TS>(zero4(), St + 16 * jt * TS::LD, qf);
            f32x4 zc = zero4();
#pragma unroll
            for (int s = 0; s <= R; ++s) zc = mma16(zc, ld_frag_tt<TK>(K, 16 * s, 16 * jt), Lf[s]);
            z[jj] = (DECAY ? zq * gp[tau + 1] : zq) + zc;
        }
    }
    // the stores after every product, so no load above waits for them
#pragma unroll
    for (int jj = 0; jj < ZJ; ++jj) {
        const int jt = cg + jj * NCG;
        if (jt < D / 16) {
            if (Zd) store4(Zd + TK::off(tau, 16 * jt + g4), z[jj]);
            if (Zwd) store4(Zwd + TK::off(tau, 16 * jt + g4), z[jj] * wz);
        }
    }
}

// a-6: fold the up-sweep nodes covering segments 0 .. seg-1 (seg > 0), or
// with p.leaf_fold the leaves 0 .. seg-1 themselves, into the state tiles acc
// that plan P gives wave w; lds_f is the staging area of the cross factors.  The same steps as the fold written out in
// hla2_forward_kernel (kept inline there: at d = 128 the compiler allocates
// registers for the call form with more spills).
template <typename T, int D, int DV, int C, bool DECAY, typename P>
__device__ __forceinline__ void hla2_fold_prefix(const FwdParams &p, int bh, int seg, float g, int w,
                                                 f32x4 (&acc)[P::NA], float *lds_f) {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    constexpr int NT = G::NT;
    using O = SumOfs<D, DV>;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    // fold node B (later) into the running state A: W <- a^2 W + N_B +
    // a S Y_B, u <- a^2 u + nv_B + a S y_B, S <- a S + X_B; the old S and
    // the node's [Y | y] are staged in LDS as the cross factors (fp32, or
    // split bf16 for the bf16 kernels at d >= 64)
    using L = CrossLds<D, DV>;  // fold: whole right factor
    using X3 = FoldX3<T, D, DV>;
    float *Ss = lds_f, *Bs = lds_f + D * L::LDA;
    bf16 *Sh = reinterpret_cast<bf16 *>(lds_f), *Sl = Sh + X3::S_EL, *Yh = Sl + X3::S_EL, *Yl = Yh + X3::Y_EL;
    int done = 0;
    while (done < seg) {
        // the next node: a leaf, or the largest up-sweep node left
        const int b = p.leaf_fold ? 0 : 31 - __builtin_clz(seg - done);
        const float *e = p.ws + node_offset(bh, b, done >> b, p.BH, p.nreal, G::SUMF);
        const float a = DECAY ? pow_int(g, (long)p.seg_len << b) : 1.f;
        // with no caller state the first node folds into zero: no cross terms
        const bool cross = p.state_in != nullptr || done > 0;
        // The node's linear parts: with d <= 64 they are loaded into
        // registers ahead of the staging, so every global load of the
        // node is in flight at once (larger heads have no registers to
        // spare)
        constexpr bool PRE = D <= 64;
        f32x4 nl[PRE ? P::NA : 1];
        auto w_lin = [&](int ti, int tv, int i) {
            return e[O::N + (16 * ti + g4 + i) * DV + 16 * tv + col];
        };
        auto u_lin = [&](int ti, int i) { return col == 0 ? e[O::nv + 16 * ti + g4 + i] : 0.f; };
        auto s_lin = [&](int ti, int tj, int i) { return e[O::X + (16 * ti + g4 + i) * D + 16 * tj + col]; };
        if constexpr (PRE) {
            for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
                for (int i = 0; i < 4; ++i) nl[j][i] = w_lin(ti, tv, i);
            });
            for_tiles<P, kU>(w, [&](int j, int ti, int) {
#pragma unroll
                for (int i = 0; i < 4; ++i) nl[j][i] = u_lin(ti, i);
            });
            for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
                for (int i = 0; i < 4; ++i) nl[j][i] = s_lin(ti, tj, i);
            });
        }
        if (cross) {
            if constexpr (X3::ON) {
                fold_x3_stage_s<P, D>(acc, w, Sh, Sl);
                fold_x3_stage_y<D, DV, NT>(Yh, Yl, e + O::Y, e + O::y, a);
            } else {
                for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) Ss[(16 * ti + g4 + i) * L::LDA + 16 * tj + col] = acc[j][i];
                });
                stage_right_ext<D, DV, DV, NT>(Bs, e + O::Y, 0, e + O::y, true);
            }
        }
        // the linear terms (the old S is already staged); the cross
        // terms once the staging has landed
        for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[j][i] = a * a * acc[j][i] + (PRE ? nl[PRE ? j : 0][i] : w_lin(ti, tv, i));
        });
        for_tiles<P, kU>(w, [&](int j, int ti, int) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = a * a * acc[j][i] + (PRE ? nl[PRE ? j : 0][i] : u_lin(ti, i));
        });
        for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[j][i] = a * acc[j][i] + (PRE ? nl[PRE ? j : 0][i] : s_lin(ti, tj, i));
        });
        if (cross) {
            __syncthreads();
            if constexpr (X3::ON) {
                fold_x3_products<P, D, DV>(acc, w, Sh, Sl, Yh, Yl);
            } else {
                for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
                    acc[j] += a * tile_ab_f32<D>(Ss + 16 * ti * L::LDA, L::LDA, Bs + 16 * tv, L::LDB);
                });
                for_tiles<P, kU>(w, [&](int j, int ti, int) {
                    acc[j] += a * tile_ab_f32<D>(Ss + 16 * ti * L::LDA, L::LDA, Bs + DV, L::LDB);
                });
            }
            __syncthreads();
        }
        done += 1 << b;
    }
}

// ------------------------------------------------------------ forward kernel

// ZO: also write the keyed queries z_t = S_t q_t of every row to p.z_out.
template <typename T, int D, int DV, int C, bool DECAY, bool ZO = false>
__global__ __launch_bounds__((Hla2Cfg<T, D, DV, C, DECAY>::NT),
                             (hla2_fwd_blocks<T, D, DV, C, DECAY>()))
void hla2_forward_kernel(FwdParams p) {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    constexpr int nTV = G::nTV;
    using TK = typename G::TK;
    using TV = typename G::TV;
    __shared__ Hla2FwdLds<T, D, DV, C, DECAY> lds;
    auto &sm = lds.s;

    int seg, bh;
    forward_slot(p, blockIdx.x, &seg, &bh);
    const int w = wave_id();
    const int r = w / NCG, cg = w % NCG;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const float g = DECAY ? p.gamma[gamma_slot(bh, p.H)] : 1.f;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const bool ratio = p.ratio != 0;
    const bool last = seg == p.nseg - 1;
    // Every wave-uniform choice inside the chunk loop is made without a
    // branch: u (the denominator's state) is always carried and the ratio's
    // products always formed, the division selected at the end.  With a
    // branch skipping those blocks, a non-ratio instance (d = 32, decay)
    // gave wrong state copies from its second chunk on, varying from run
    // to run; the branch-free loop is exact.
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * p.n * DV;
    const __amdgpu_buffer_rsrc_t orsrc = rows_rsrc(o + (size_t)t_begin * DV, t_end - t_begin, DV);
    T *zo = ZO ? static_cast<T *>(p.z_out) + ((size_t)bh * p.n + t_begin) * D : nullptr;
    const __amdgpu_buffer_rsrc_t zrsrc = rows_rsrc(zo, ZO ? t_end - t_begin : 0, D);
    using TO = typename G::TO;
    constexpr bool RO = hla2_rows_out<T, D, DV, C, DECAY>();
    T *const ot = sm.Ot + (RO ? w * 16 * TO::LD : 0);   // this wave's staging rows

    // the next chunk's data in registers: K, V for LDS; this wave's Q rows
    ChunkRegs<T, C, D, NT> rk;
    ChunkRegs<T, C, DV, NT> rv;
    RowFrags<T, D> qn;
    auto load_chunk = [&](int c, int valid) {
        const int tv = valid - 16 * r;     // valid rows of this wave's tile
        qn.load_rows_g(q + (size_t)(c + (tv > 0 ? 16 * r : 0)) * D, D, tv > 0 ? tv : 0);
        rk.load(k + (size_t)c * D, valid);
        rv.load(v + (size_t)c * DV, valid);
    };

    // ---- a-6 / a-7: carried state at the start of this segment: the caller's
    // state (or zero), then the up-sweep nodes covering segments 0 .. seg-1
    const float *S0 = nullptr, *W0 = nullptr, *u0 = nullptr;
    if (p.state_in) {
        const float *e = p.state_in + (size_t)bh * G::STF;
        S0 = e;
        W0 = e + D * D;
        u0 = e + D * D + D * DV;
    }
    using O = SumOfs<D, DV>;

    // Everything below runs unrolled for the wave's row tile R, so each wave
    // holds exactly the state tiles its plan gives it.
    with_row_tile<RT>(r, [&](auto rt) {
        constexpr int R = decltype(rt)::value;
        using P = typename G::template FwdPlan<R>;
        const int tau = 16 * R + col;    // the lane's token within the chunk

        // the fp32 state tiles this wave holds (u as column tile nTV of W)
        f32x4 acc[P::NA];
        for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = S0 ? S0[(16 * ti + g4 + i) * D + 16 * tj + col] : 0.f;
        });
        for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = W0 ? W0[(16 * ti + g4 + i) * DV + 16 * tv + col] : 0.f;
        });
        for_tiles<P, kU>(w, [&](int j, int ti, int) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = (u0 && col == 0) ? u0[16 * ti + g4 + i] : 0.f;
        });
        if (seg > 0) {
            // fold node B (later) into the running state A: W <- a^2 W + N_B +
            // a S Y_B, u <- a^2 u + nv_B + a S y_B, S <- a S + X_B; the old S and
            // the node's [Y | y] are staged in LDS as the cross factors (fp32,
            // or split bf16 for the bf16 kernels at d >= 64)
            using L = CrossLds<D, DV>;  // fold: whole right factor
            using X3 = FoldX3<T, D, DV>;
            float *Ss = lds.f, *Bs = lds.f + D * L::LDA;
            bf16 *Sh = reinterpret_cast<bf16 *>(lds.f), *Sl = Sh + X3::S_EL, *Yh = Sl + X3::S_EL,
                 *Yl = Yh + X3::Y_EL;
            int done = 0;
            while (done < seg) {
                // the next node: a leaf, or the largest up-sweep node left
                const int b = p.leaf_fold ? 0 : 31 - __builtin_clz(seg - done);
                const float *e = p.ws + node_offset(bh, b, done >> b, p.BH, p.nreal, G::SUMF);
                const float a = DECAY ? pow_int(g, (long)p.seg_len << b) : 1.f;
                // with no caller state the first node folds into zero: no cross terms
                const bool cross = p.state_in != nullptr || done > 0;
                // The node's linear parts: with d <= 64 they are loaded into
                // registers ahead of the staging, so every global load of the
                // node is in flight at once (larger heads have no registers to
                // spare)
                constexpr bool PRE = D <= 64;
                f32x4 nl[PRE ? P::NA : 1];
                auto w_lin = [&](int ti, int tv, int i) {
                    return e[O::N + (16 * ti + g4 + i) * DV + 16 * tv + col];
                };
                auto u_lin = [&](int ti, int i) { return col == 0 ? e[O::nv + 16 * ti + g4 + i] : 0.f; };
                auto s_lin = [&](int ti, int tj, int i) { return e[O::X + (16 * ti + g4 + i) * D + 16 * tj + col]; };
                if constexpr (PRE) {
                    for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) nl[j][i] = w_lin(ti, tv, i);
                    });
                    for_tiles<P, kU>(w, [&](int j, int ti, int) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) nl[j][i] = u_lin(ti, i);
                    });
                    for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) nl[j][i] = s_lin(ti, tj, i);
                    });
                }
                if (cross) {
                    if constexpr (X3::ON) {
                        fold_x3_stage_s<P, D>(acc, w, Sh, Sl);
                        fold_x3_stage_y<D, DV, NT>(Yh, Yl, e + O::Y, e + O::y, a);
                    } else {
                        for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) Ss[(16 * ti + g4 + i) * L::LDA + 16 * tj + col] = acc[j][i];
                        });
                        stage_right_ext<D, DV, DV, NT>(Bs, e + O::Y, 0, e + O::y, true);
                    }
                }
                // the linear terms (the old S is already staged); the cross
                // terms once the staging has landed
                for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[j][i] = a * a * acc[j][i] + (PRE ? nl[PRE ? j : 0][i] : w_lin(ti, tv, i));
                });
                for_tiles<P, kU>(w, [&](int j, int ti, int) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j][i] = a * a * acc[j][i] + (PRE ? nl[PRE ? j : 0][i] : u_lin(ti, i));
                });
                for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[j][i] = a * acc[j][i] + (PRE ? nl[PRE ? j : 0][i] : s_lin(ti, tj, i));
                });
                if (cross) {
                    __syncthreads();
                    if constexpr (X3::ON) {
                        fold_x3_products<P, D, DV>(acc, w, Sh, Sl, Yh, Yl);
                    } else {
                        for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
                            acc[j] += a * tile_ab_f32<D>(Ss + 16 * ti * L::LDA, L::LDA, Bs + 16 * tv, L::LDB);
                        });
                        for_tiles<P, kU>(w, [&](int j, int ti, int) {
                            acc[j] += a * tile_ab_f32<D>(Ss + 16 * ti * L::LDA, L::LDA, Bs + DV, L::LDB);
                        });
                    }
                    __syncthreads();
                }
                done += 1 << b;
            }
        }
        // T-typed transposed copies: the operands of Q S0 and Q W0 (row DV of Wt = u)
        auto store_copies = [&](bool with_u) {
            for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
                store4(sm.St + G::TS::off(16 * tj + col, 16 * ti + g4), acc[j]);
            });
            for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
                store4(sm.Wt + G::TS::off(16 * tv + col, 16 * ti + g4), acc[j]);
            });
            if (with_u) {
                for_tiles<P, kU>(w, [&](int j, int ti, int) {
                    store4(sm.Wt + G::TS::off(DV + col, 16 * ti + g4), acc[j]);
                });
            }
        };
        store_copies(true);
        if (DECAY) fill_pow_table<NT>(sm.gp, G::NPOW, g);

        int c0 = t_begin;
        int cv = min(C, t_end - c0);
        load_chunk(c0, cv);

        while (c0 < t_end) {
            __syncthreads();   // previous chunk's readers are done; setup is visible
            // ---- a-1: stage this chunk, then start loading the next one
            rk.template store_tile<TK>(sm.K);
            if (DECAY) rk.template store_tile_w<TK>(sm.Kw, sm.gp, cv - 1);
            rv.template store_tile<TV>(sm.V);
            RowFrags<T, D> qf = qn;            // the row tile's Q: operand of four products
            qf.mask_rows(cv - 16 * R);
            const int n0 = c0 + C;
            const int ncv = min(C, t_end - n0);
            if (n0 < t_end) load_chunk(n0, ncv);
            __syncthreads();

            // ---- a-7: advance the held state tiles of phase PH by this chunk
            const float gc = DECAY ? sm.gp[cv] : 1.f;
            const float gc2 = DECAY ? sm.gp[2 * cv] : 1.f;
            const T *KA = DECAY ? sm.Kw : sm.K;
            const T *ZA = DECAY ? sm.Zw : sm.Z;
            auto advance = [&](auto ph) {
                for_groups<P, -1, decltype(ph)::value>(w, [&](auto gi, int ti0, int tj0) {
                    constexpr Grp gr = P::grp(decltype(gi)::value);
                    f32x4 *a = acc + gr.first;
                    if constexpr (gr.mat == kS) {
                        if (DECAY) {
#pragma unroll
                            for (int x = 0; x < gr.nr * gr.nc; ++x) a[x] *= gc;
                        }
                        mma_tn_grp<gr.nr, gr.nc, C, TK, TK, false>(a, KA, 16 * ti0, sm.K, 16 * tj0);
                    } else {
                        if (DECAY) {
#pragma unroll
                            for (int x = 0; x < gr.nr * gr.nc; ++x) a[x] *= gc2;
                        }
                        mma_tn_grp<gr.nr, gr.nc, C, TK, TV, gr.mat == kU>(a, ZA, 16 * ti0, sm.V, 16 * tj0);
                    }
                });
            };

            // ---- a-2: L^T for this row tile, as operand fragments
            Frag16<T> Lf[R + 1];
            scores_t<T, D, R, TK, DECAY>(Lf, sm.K, qf, tau, sm.gp, 1);

            // ---- a-3: Z^T = diag(g^(tau+1)) (Q S0)^T + K^T L^T
            const float wz = DECAY ? (tau < cv ? sm.gp[2 * (cv - 1 - tau)] : 0.f) : 1.f;
            z_tiles<T, D, R, NCG, G::ZJ, TK, DECAY, typename G::TS>(qf, Lf, sm.St, sm.K, sm.Z,
                                                                     DECAY ? sm.Zw : nullptr, wz, sm.gp, cg, tau);
            // ---- a-4 (carried part): O^T = diag(g^(2(tau+1))) (Q W0)^T; the
            // denominator's carried part q . u0 is row DV of the widened product
            f32x4 accO[G::OJ];
#pragma unroll
            for (int jj = 0; jj < G::OJ; ++jj) {
                const int jv = RO ? cg * G::OJ + jj : cg + jj * NCG;
                accO[jj] = zero4();
                if (jv < nTV) {
                    accO[jj] = mma_nt_ft<typename G::TS>(zero4(), sm.Wt + 16 * jv * G::TS::LD, qf);
                    if (DECAY) accO[jj] *= sm.gp[2 * (tau + 1)];
                }
            }
            f32x4 accD = mma_nt_ft<typename G::TS>(zero4(), sm.Wt + DV * G::TS::LD, qf);
            if (DECAY) accD *= sm.gp[2 * (tau + 1)];
            // products of the staged chunk alone (S += K^T K), while the waves
            // of later row tiles finish Z
            advance(std::integral_constant<int, 0>{});
            __syncthreads();

            // ---- a-4: P^T = (D_{g^2} * tril(Q Z^T))^T ; O^T += V^T P^T
            Frag16<T> Pf[R + 1];
            scores_t<T, D, R, TK, DECAY>(Pf, sm.Z, qf, tau, sm.gp, 2);
            // den = q . u0 + P 1: the product with a ones column tile puts
            // P 1 in slot 0 of the token's lane in group 0
            f32x4 dc = zero4();
            const Frag16<T> ones = ones_frag<T>();
#pragma unroll
            for (int s = 0; s <= R; ++s) dc = mma16(dc, ones, Pf[s]);
            const float den = __shfl(accD[0] + dc[0], col);
            const float rden = ratio ? 1.f / den : 1.f;
#pragma unroll
            for (int jj = 0; jj < G::OJ; ++jj) {
                const int jv = RO ? cg * G::OJ + jj : cg + jj * NCG;
                if (jv < nTV) {
                    f32x4 oc = zero4();
#pragma unroll
                    for (int s = 0; s <= R; ++s)
                        oc = mma16(oc, ld_frag_tt<TV>(sm.V, 16 * s, 16 * jv), Pf[s]);
                    const f32x4 ov = (accO[jj] + oc) * rden;
                    if constexpr (RO) store4(ot + TO::off(col, 16 * jj + g4), ov);
                    else store4_row<T>(orsrc, ((c0 - t_begin + tau) * DV + 16 * jv + g4) * (int)sizeof(T), ov);
                }
            }
            if constexpr (RO)
                store_rows_out<T, TO, DV / NCG, DV>(ot, orsrc, c0 - t_begin + 16 * R, cg * (DV / NCG));
            // the keyed queries, whole in Z since the barrier above: this
            // wave's rows, its column group's share of them
            if constexpr (ZO)
                copy_rows_out<T, TK, D / NCG, D>(sm.Z, zrsrc, 16 * R, c0 - t_begin + 16 * R, cg * (D / NCG));

            // the rest of the state (W, u: products of Z) after every product,
            // then the T-typed copies, so no operand load waits behind a store
            advance(std::integral_constant<int, 1>{});
            store_copies(true);
            c0 = n0;
            cv = ncv;
        }

        if (p.state_out && last) {
            float *so = p.state_out + (size_t)bh * G::STF;
            for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
                for (int i = 0; i < 4; ++i) so[(16 * ti + g4 + i) * D + 16 * tj + col] = acc[j][i];
            });
            for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
                for (int i = 0; i < 4; ++i) so[D * D + (16 * ti + g4 + i) * DV + 16 * tv + col] = acc[j][i];
            });
            for_tiles<P, kU>(w, [&](int j, int ti, int) {
                if (col == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) so[D * D + D * DV + 16 * ti + g4 + i] = acc[j][i];
                }
            });
        }
    });
}

// ------------------------------------------------------------ summary kernel

template <typename T, int D, int DV, int C, bool DECAY>
__global__ __launch_bounds__((Hla2Cfg<T, D, DV, C, DECAY>::NT),
                             (hla2_sum_blocks<T, D, DV, C, DECAY>()))
void hla2_summary_kernel(FwdParams p) {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    using TK = typename G::TK;
    using TV = typename G::TV;
    __shared__ Hla2SumSmem<T, D, DV, C, DECAY> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
    const int r = w / NCG, cg = w % NCG;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const float g = DECAY ? p.gamma[gamma_slot(bh, p.H)] : 1.f;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;

    if (DECAY) fill_pow_table<NT>(sm.gp, G::NPOW, g);
    for (int i = threadIdx.x; i < D * G::TS::LD; i += NT) sm.St[i] = from_f<T>(0.f);

    ChunkRegs<T, C, D, NT> rq, rk;
    ChunkRegs<T, C, DV, NT> rv;

    // Everything below runs unrolled for the wave's row tile R, so each wave
    // holds exactly the summary tiles its plan gives it.
    with_row_tile<RT>(r, [&](auto rt) {
        constexpr int R = decltype(rt)::value;
        using P = typename G::template SumPlan<R>;
        const int tau = 16 * R + col;
        // S, W, C and the stripes u = Z^T 1, m = Q^T 1, all from zero
        f32x4 acc[P::NA];
#pragma unroll
        for (int j = 0; j < P::NA; ++j) acc[j] = zero4();

        int c0 = t_begin;
        int cv = min(C, t_end - c0);
        rq.load(q + (size_t)c0 * D, cv);
        rk.load(k + (size_t)c0 * D, cv);
        rv.load(v + (size_t)c0 * DV, cv);

        while (c0 < t_end) {
            __syncthreads();
            rq.template store_tile<TK>(sm.Q);
            if (DECAY) rq.template store_tile_w<TK>(sm.Qw, sm.gp, cv - 1);
            rk.template store_tile<TK>(sm.K);
            if (DECAY) rk.template store_tile_w<TK>(sm.Kw, sm.gp, cv - 1);
            rv.template store_tile<TV>(sm.V);
            const int n0 = c0 + C;
            const int ncv = min(C, t_end - n0);
            if (n0 < t_end) {
                rq.load(q + (size_t)n0 * D, ncv);
                rk.load(k + (size_t)n0 * D, ncv);
                rv.load(v + (size_t)n0 * DV, ncv);
            }
            __syncthreads();

            const float gc = DECAY ? sm.gp[cv] : 1.f;
            const float gc2 = DECAY ? sm.gp[2 * cv] : 1.f;
            const T *KA = DECAY ? sm.Kw : sm.K;
            const T *QA = DECAY ? sm.Qw : sm.Q;
            // advance the held tiles of phase PH by this chunk: S += K^T K,
            // C (m) += Q^T [V | 1], W (u) += Z^T [V | 1]
            auto advance = [&](auto ph) {
                for_groups<P, -1, decltype(ph)::value>(w, [&](auto gi, int ti0, int tj0) {
                    constexpr Grp gr = P::grp(decltype(gi)::value);
                    f32x4 *a = acc + gr.first;
                    const float sc = (gr.mat == kW || gr.mat == kU) ? gc2 : gc;
                    if (DECAY) {
#pragma unroll
                        for (int x = 0; x < gr.nr * gr.nc; ++x) a[x] *= sc;
                    }
                    if constexpr (gr.mat == kS)
                        mma_tn_grp<gr.nr, gr.nc, C, TK, TK, false>(a, KA, 16 * ti0, sm.K, 16 * tj0);
                    else if constexpr (gr.mat == kW || gr.mat == kU)
                        mma_tn_grp<gr.nr, gr.nc, C, TK, TV, gr.mat == kU>(a, sm.Z, 16 * ti0, sm.V, 16 * tj0);
                    else
                        mma_tn_grp<gr.nr, gr.nc, C, TK, TV, gr.mat == kM>(a, QA, 16 * ti0, sm.V, 16 * tj0);
                });
            };

            RowFrags<T, D> qf;
            qf.template load_t<TK>(sm.Q + 16 * R * TK::LD);
            Frag16<T> Lf[R + 1];
            scores_t<T, D, R, TK, DECAY>(Lf, sm.K, qf, tau, sm.gp, 1);
            // Z rows weighted by g^(2(c-1-tau)): only the W and u updates use Z here
            const float wz = tau < cv ? (DECAY ? sm.gp[2 * (cv - 1 - tau)] : 1.f) : 0.f;
            z_tiles<T, D, R, NCG, G::ZJ, TK, DECAY, typename G::TS>(qf, Lf, sm.St, sm.K, nullptr, sm.Z, wz, sm.gp,
                                                                     cg, tau);
            // products of the staged chunk alone, while later row tiles finish Z
            advance(std::integral_constant<int, 0>{});
            __syncthreads();
            advance(std::integral_constant<int, 1>{});
            // the running S's T-typed copy after every product of the chunk
            for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
                store4(sm.St + G::TS::off(16 * tj + col, 16 * ti + g4), acc[j]);
            });
            c0 = n0;
            cv = ncv;
        }

        // summary [X = S | Y = C | N = W | y = m | nv = u]
        float *e = p.ws + node_offset(bh, 0, seg, p.BH, p.nreal, G::SUMF);
        for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
            for (int i = 0; i < 4; ++i) e[(16 * ti + g4 + i) * D + 16 * tj + col] = acc[j][i];
        });
        for_tiles<P, kC>(w, [&](int j, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) e[D * D + (16 * ti + g4 + i) * DV + 16 * tv + col] = acc[j][i];
        });
        for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) e[D * D + D * DV + (16 * ti + g4 + i) * DV + 16 * tv + col] = acc[j][i];
        });
        for_tiles<P, kM>(w, [&](int j, int ti, int) {
            if (col == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) e[D * D + 2 * D * DV + 16 * ti + g4 + i] = acc[j][i];
            }
        });
        for_tiles<P, kU>(w, [&](int j, int ti, int) {
            if (col == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) e[D * D + 2 * D * DV + D + 16 * ti + g4 + i] = acc[j][i];
            }
        });
    });
}

}  // namespace hla
