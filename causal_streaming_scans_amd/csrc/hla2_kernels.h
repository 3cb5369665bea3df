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
// token, so the output is written straight from registers.  Z goes through
// LDS (row-major for P, and decay-weighted transposed for the W update),
// since every row tile needs all earlier rows of it.  The fp32 state S0, W0
// is spread over all waves as MFMA accumulators for the whole segment; its
// T-typed transposed copy in LDS is the operand of Q S0 and Q W0.  The next
// chunk's Q, K, V are loaded into registers while the current one computes.
#pragma once

#include "chunk_common.h"

namespace hla {

template <typename T, int D, int DV, int C, bool DECAY>
struct Hla2Cfg {
    using WS = WaveShape<C, D>;
    static constexpr int RT = WS::RT, NCG = WS::NCG, NW = WS::NW, NT = WS::NT;
    static constexpr int LDD = ld_of<T>(D);   // rows of length D
    static constexpr int LDC = ld_of<T>(C);   // rows of length C
    static constexpr int nTD = D / 16, nTV = DV / 16;
    static constexpr int ZJ = (nTD + NCG - 1) / NCG;    // Z^T tiles per wave
    static constexpr int OJ = (nTV + NCG - 1) / NCG;    // O^T tiles per wave
    using SB = TileBlocks<nTD, nTD, NW>;    // ownership of S tiles
    using WB = TileBlocks<nTD, nTV, NW>;    // ownership of W (and C) tiles
    static constexpr int SUMF = summary_floats(D, DV);
    static constexpr int STF = hla2_state_floats(D, DV);
    static constexpr int NPOW = 2 * C + 2;
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

template <typename T, int D, int DV, int C, bool DECAY>
struct Hla2FwdSmem {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T K[C * G::LDD];
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Ktw[DECAY ? D * G::LDC : 8];   // K^T weighted by g^(c-1-tau)
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T Z[C * G::LDD];
    alignas(16) T Ztw[D * G::LDC];               // Z^T weighted by g^(2(c-1-tau))
    alignas(16) T St[D * G::LDD];                // St[j][i] = S0[i][j]
    alignas(16) T Wt[DV * G::LDD];               // Wt[j][i] = W0[i][j]
    float u0[D];
    float gp[G::NPOW];
};

template <typename T, int D, int DV, int C, bool DECAY>
struct Hla2SumSmem {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T K[C * G::LDD];
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Ktw[DECAY ? D * G::LDC : 8];
    alignas(16) T Qtw[D * G::LDC];               // Q^T weighted by g^(c-1-tau)
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T Ztw[D * G::LDC];
    alignas(16) T St[D * G::LDD];
    float u0[D];
    float m0[D];
    float gp[G::NPOW];
};

template <int NT, int NW, int D, int DV>
constexpr int hla2_min_blocks() {
    return (D <= 64 && DV <= 64 && NT <= 256) ? 2 : 1;
}

// L^T tiles of row tile r as operand fragments: Lf[s] holds
// (D_g * tril(Q K^T))^T[sigma in tile s][tau in tile r], s <= r.
template <typename T, int D, int RT, int LDD, bool DECAY>
__device__ __forceinline__ void scores_t(Frag16<T> (&Lf)[RT], const T *K, const RowFrags<T, D> &qf,
                                         int r, int tau, const float *gp, int gexp) {
    const int g4 = (lane_id() >> 4) << 2;
#pragma unroll
    for (int s = 0; s < RT; ++s) {
        if (s <= r) {
            f32x4 a = mma_nt_f(zero4(), K + 16 * s * LDD, LDD, qf);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sigma = 16 * s + g4 + i;
                float m = 0.f;
                if (sigma <= tau) m = DECAY ? a[i] * gp[gexp * (tau - sigma)] : a[i];
                a[i] = m;
            }
            Lf[s] = to_frag<T>(a);
        }
    }
}

// ------------------------------------------------------------ forward kernel

template <typename T, int D, int DV, int C, bool DECAY>
__global__ __launch_bounds__((Hla2Cfg<T, D, DV, C, DECAY>::NT),
                             (hla2_min_blocks<Hla2Cfg<T, D, DV, C, DECAY>::NT, 0, D, DV>()))
void hla2_forward_kernel(FwdParams p) {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    constexpr int LDD = G::LDD, LDC = G::LDC, nTD = G::nTD, nTV = G::nTV;
    __shared__ Hla2FwdSmem<T, D, DV, C, DECAY> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
    const int r = w / NCG, cg = w % NCG;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const int tau = 16 * r + col;          // the lane's token within the chunk
    const float g = DECAY ? p.gamma[bh % p.H] : 1.f;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * p.n * DV;

    if (DECAY) fill_pow_table<NT>(sm.gp, G::NPOW, g);

    // carried state at the start of this segment: the exclusive prefix from
    // the scan, or the caller's state, or zero
    const float *S0 = nullptr, *W0 = nullptr, *u0 = nullptr;
    if (p.nseg > 1) {
        const float *e = p.ws + ws_elem(bh, 1, p.spad, seg, G::SUMF);
        S0 = e;
        W0 = e + D * D + D * DV;
        u0 = e + D * D + 2 * D * DV + D;
    } else if (p.state_in) {
        const float *e = p.state_in + (size_t)bh * G::STF;
        S0 = e;
        W0 = e + D * D;
        u0 = e + D * D + D * DV;
    }
    using SB = typename G::SB;
    using WB = typename G::WB;
    f32x4 accS[SB::PB][SB::BR][SB::BR], accW[WB::PB][WB::BR][WB::BR];
    for_owned<SB, NW>(w, [&](int pb, int x, int y, int ti, int tj) {
        f32x4 a;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = S0 ? S0[(16 * ti + g4 + i) * D + 16 * tj + col] : 0.f;
        accS[pb][x][y] = a;
        store4(sm.St + (16 * tj + col) * LDD + 16 * ti + g4, a);
    });
    for_owned<WB, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
        f32x4 a;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = W0 ? W0[(16 * ti + g4 + i) * DV + 16 * tv + col] : 0.f;
        accW[pb][x][y] = a;
        store4(sm.Wt + (16 * tv + col) * LDD + 16 * ti + g4, a);
    });
    for (int i = threadIdx.x; i < D; i += NT) sm.u0[i] = u0 ? u0[i] : 0.f;

    ChunkRegs<T, C, D, NT> rq, rk;
    ChunkRegs<T, C, DV, NT> rv;
    int c0 = t_begin;
    int cv = min(C, t_end - c0);
    rq.load(q + (size_t)c0 * D, cv);
    rk.load(k + (size_t)c0 * D, cv);
    rv.load(v + (size_t)c0 * DV, cv);

    while (c0 < t_end) {
        __syncthreads();   // previous chunk's readers are done; setup is visible
        // ---- a-1: stage this chunk, then start loading the next one
        rq.store_rows(sm.Q, LDD);
        rk.store_rows(sm.K, LDD);
        rk.store_cols(sm.Kt, LDC);
        if (DECAY) rk.store_cols_w(sm.Ktw, LDC, sm.gp, cv - 1);
        rv.store_cols(sm.Vt, LDC);
        const int n0 = c0 + C;
        const int ncv = min(C, t_end - n0);
        if (n0 < t_end) {
            rq.load(q + (size_t)n0 * D, ncv);
            rk.load(k + (size_t)n0 * D, ncv);
            rv.load(v + (size_t)n0 * DV, ncv);
        }
        __syncthreads();

        // the row tile's Q, kept in registers: an operand of four products
        RowFrags<T, D> qf;
        qf.load(sm.Q + 16 * r * LDD, LDD);
        // ---- a-2: L^T for this row tile, as operand fragments
        Frag16<T> Lf[RT];
        scores_t<T, D, RT, LDD, DECAY>(Lf, sm.K, qf, r, tau, sm.gp, 1);

        // ---- a-3: Z^T = diag(g^(tau+1)) (Q S0)^T + K^T L^T
        const float wz = tau < cv ? (DECAY ? sm.gp[2 * (cv - 1 - tau)] : 1.f) : 0.f;
#pragma unroll
        for (int jj = 0; jj < G::ZJ; ++jj) {
            const int jt = cg + jj * NCG;
            if (jt < nTD) {
                f32x4 z = mma_nt_f(zero4(), sm.St + 16 * jt * LDD, LDD, qf);
                f32x4 zc = zero4();
#pragma unroll
                for (int s = 0; s < RT; ++s)
                    if (s <= r) zc = mma16(zc, ld_frag(sm.Kt + 16 * jt * LDC + 16 * s, LDC), Lf[s]);
                z = (DECAY ? z * sm.gp[tau + 1] : z) + zc;
                store4(sm.Z + tau * LDD + 16 * jt + g4, z);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.Ztw[(16 * jt + g4 + i) * LDC + tau] = from_f<T>(z[i] * wz);
            }
        }
        // ---- a-4 (carried part): O^T = diag(g^(2(tau+1))) (Q W0)^T, den = that for u0
        f32x4 accO[G::OJ];
#pragma unroll
        for (int jj = 0; jj < G::OJ; ++jj) {
            const int jv = cg + jj * NCG;
            accO[jj] = zero4();
            if (jv < nTV) {
                accO[jj] = mma_nt_f(zero4(), sm.Wt + 16 * jv * LDD, LDD, qf);
                if (DECAY) accO[jj] *= sm.gp[2 * (tau + 1)];
            }
        }
        float den = 0.f;
        if (p.ratio) {
            den = lane_dot<T, D>(sm.Q + tau * LDD, sm.u0);
            if (DECAY) den *= sm.gp[2 * (tau + 1)];
        }
        __syncthreads();

        // ---- a-4: P^T = (D_{g^2} * tril(Q Z^T))^T ; O^T += V^T P^T
        Frag16<T> Pf[RT];
        scores_t<T, D, RT, LDD, DECAY>(Pf, sm.Z, qf, r, tau, sm.gp, 2);
        if (p.ratio) {
            float rs = 0.f;
#pragma unroll
            for (int s = 0; s < RT; ++s)
                if (s <= r) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) rs += frag_val(Pf[s], i);
                }
            den += sum_groups(rs);
        }
#pragma unroll
        for (int jj = 0; jj < G::OJ; ++jj) {
            const int jv = cg + jj * NCG;
            if (jv < nTV) {
                f32x4 oc = zero4();
#pragma unroll
                for (int s = 0; s < RT; ++s)
                    if (s <= r) oc = mma16(oc, ld_frag(sm.Vt + 16 * jv * LDC + 16 * s, LDC), Pf[s]);
                f32x4 ov = accO[jj] + oc;
                if (p.ratio) ov *= 1.f / den;
                if (tau < cv) store4(o + (size_t)(c0 + tau) * DV + 16 * jv + g4, ov);
            }
        }

        // ---- a-7: advance the carried state by this chunk
        const float gc = DECAY ? sm.gp[cv] : 1.f;
        const float gc2 = DECAY ? sm.gp[2 * cv] : 1.f;
        const T *KA = DECAY ? sm.Ktw : sm.Kt;
        for_blocks<SB, NW>(w, [&](int pb, int ti0, int tj0) {
            if (DECAY) {
#pragma unroll
                for (int x = 0; x < SB::BR; ++x)
#pragma unroll
                    for (int y = 0; y < SB::BR; ++y) accS[pb][x][y] *= gc;
            }
            mma_nt_blk<SB::BR, C>(accS[pb], KA + 16 * ti0 * LDC, LDC, sm.Kt + 16 * tj0 * LDC, LDC);
#pragma unroll
            for (int x = 0; x < SB::BR; ++x)
#pragma unroll
                for (int y = 0; y < SB::BR; ++y)
                    store4(sm.St + (16 * (tj0 + y) + col) * LDD + 16 * (ti0 + x) + g4, accS[pb][x][y]);
        });
        for_blocks<WB, NW>(w, [&](int pb, int ti0, int tv0) {
            if (DECAY) {
#pragma unroll
                for (int x = 0; x < WB::BR; ++x)
#pragma unroll
                    for (int y = 0; y < WB::BR; ++y) accW[pb][x][y] *= gc2;
            }
            mma_nt_blk<WB::BR, C>(accW[pb], sm.Ztw + 16 * ti0 * LDC, LDC, sm.Vt + 16 * tv0 * LDC, LDC);
#pragma unroll
            for (int x = 0; x < WB::BR; ++x)
#pragma unroll
                for (int y = 0; y < WB::BR; ++y)
                    store4(sm.Wt + (16 * (tv0 + y) + col) * LDD + 16 * (ti0 + x) + g4, accW[pb][x][y]);
        });
        for (int i = threadIdx.x; i < D; i += NT)
            sm.u0[i] = gc2 * sm.u0[i] + row_sum<T, C>(sm.Ztw, LDC, i);
        c0 = n0;
        cv = ncv;
    }

    if (p.state_out && seg == p.nseg - 1) {
        float *so = p.state_out + (size_t)bh * G::STF;
        for_owned<SB, NW>(w, [&](int pb, int x, int y, int ti, int tj) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[(16 * ti + g4 + i) * D + 16 * tj + col] = accS[pb][x][y][i];
        });
        for_owned<WB, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[D * D + (16 * ti + g4 + i) * DV + 16 * tv + col] = accW[pb][x][y][i];
        });
        __syncthreads();
        for (int i = threadIdx.x; i < D; i += NT) so[D * D + D * DV + i] = sm.u0[i];
    }
}

// ------------------------------------------------------------ summary kernel

template <typename T, int D, int DV, int C, bool DECAY>
__global__ __launch_bounds__((Hla2Cfg<T, D, DV, C, DECAY>::NT),
                             (hla2_min_blocks<Hla2Cfg<T, D, DV, C, DECAY>::NT, 0, D, DV>()))
void hla2_summary_kernel(FwdParams p) {
    using G = Hla2Cfg<T, D, DV, C, DECAY>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    constexpr int LDD = G::LDD, LDC = G::LDC, nTD = G::nTD, nTV = G::nTV;
    __shared__ Hla2SumSmem<T, D, DV, C, DECAY> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
    const int r = w / NCG, cg = w % NCG;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const int tau = 16 * r + col;
    const float g = DECAY ? p.gamma[bh % p.H] : 1.f;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;

    if (DECAY) fill_pow_table<NT>(sm.gp, G::NPOW, g);
    using SB = typename G::SB;
    using WB = typename G::WB;
    f32x4 accS[SB::PB][SB::BR][SB::BR], accW[WB::PB][WB::BR][WB::BR], accC[WB::PB][WB::BR][WB::BR];
#pragma unroll
    for (int pb = 0; pb < SB::PB; ++pb)
#pragma unroll
        for (int x = 0; x < SB::BR; ++x)
#pragma unroll
            for (int y = 0; y < SB::BR; ++y) accS[pb][x][y] = zero4();
#pragma unroll
    for (int pb = 0; pb < WB::PB; ++pb)
#pragma unroll
        for (int x = 0; x < WB::BR; ++x)
#pragma unroll
            for (int y = 0; y < WB::BR; ++y) {
                accW[pb][x][y] = zero4();
                accC[pb][x][y] = zero4();
            }
    for (int i = threadIdx.x; i < D * LDD; i += NT) sm.St[i] = from_f<T>(0.f);
    for (int i = threadIdx.x; i < D; i += NT) {
        sm.u0[i] = 0.f;
        sm.m0[i] = 0.f;
    }

    ChunkRegs<T, C, D, NT> rq, rk;
    ChunkRegs<T, C, DV, NT> rv;
    int c0 = t_begin;
    int cv = min(C, t_end - c0);
    rq.load(q + (size_t)c0 * D, cv);
    rk.load(k + (size_t)c0 * D, cv);
    rv.load(v + (size_t)c0 * DV, cv);

    while (c0 < t_end) {
        __syncthreads();
        rq.store_rows(sm.Q, LDD);
        if (DECAY) rq.store_cols_w(sm.Qtw, LDC, sm.gp, cv - 1);
        else rq.store_cols(sm.Qtw, LDC);
        rk.store_rows(sm.K, LDD);
        rk.store_cols(sm.Kt, LDC);
        if (DECAY) rk.store_cols_w(sm.Ktw, LDC, sm.gp, cv - 1);
        rv.store_cols(sm.Vt, LDC);
        const int n0 = c0 + C;
        const int ncv = min(C, t_end - n0);
        if (n0 < t_end) {
            rq.load(q + (size_t)n0 * D, ncv);
            rk.load(k + (size_t)n0 * D, ncv);
            rv.load(v + (size_t)n0 * DV, ncv);
        }
        __syncthreads();

        RowFrags<T, D> qf;
        qf.load(sm.Q + 16 * r * LDD, LDD);
        Frag16<T> Lf[RT];
        scores_t<T, D, RT, LDD, DECAY>(Lf, sm.K, qf, r, tau, sm.gp, 1);
        const float wz = tau < cv ? (DECAY ? sm.gp[2 * (cv - 1 - tau)] : 1.f) : 0.f;
#pragma unroll
        for (int jj = 0; jj < G::ZJ; ++jj) {
            const int jt = cg + jj * NCG;
            if (jt < nTD) {
                f32x4 z = mma_nt_f(zero4(), sm.St + 16 * jt * LDD, LDD, qf);
                f32x4 zc = zero4();
#pragma unroll
                for (int s = 0; s < RT; ++s)
                    if (s <= r) zc = mma16(zc, ld_frag(sm.Kt + 16 * jt * LDC + 16 * s, LDC), Lf[s]);
                z = (DECAY ? z * sm.gp[tau + 1] : z) + zc;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.Ztw[(16 * jt + g4 + i) * LDC + tau] = from_f<T>(z[i] * wz);
            }
        }
        __syncthreads();

        const float gc = DECAY ? sm.gp[cv] : 1.f;
        const float gc2 = DECAY ? sm.gp[2 * cv] : 1.f;
        const T *KA = DECAY ? sm.Ktw : sm.Kt;
        for_blocks<SB, NW>(w, [&](int pb, int ti0, int tj0) {
            if (DECAY) {
#pragma unroll
                for (int x = 0; x < SB::BR; ++x)
#pragma unroll
                    for (int y = 0; y < SB::BR; ++y) accS[pb][x][y] *= gc;
            }
            mma_nt_blk<SB::BR, C>(accS[pb], KA + 16 * ti0 * LDC, LDC, sm.Kt + 16 * tj0 * LDC, LDC);
#pragma unroll
            for (int x = 0; x < SB::BR; ++x)
#pragma unroll
                for (int y = 0; y < SB::BR; ++y)
                    store4(sm.St + (16 * (tj0 + y) + col) * LDD + 16 * (ti0 + x) + g4, accS[pb][x][y]);
        });
        for_blocks<WB, NW>(w, [&](int pb, int ti0, int tv0) {
            if (DECAY) {
#pragma unroll
                for (int x = 0; x < WB::BR; ++x)
#pragma unroll
                    for (int y = 0; y < WB::BR; ++y) {
                        accW[pb][x][y] *= gc2;
                        accC[pb][x][y] *= gc;
                    }
            }
            mma_nt_blk<WB::BR, C>(accW[pb], sm.Ztw + 16 * ti0 * LDC, LDC, sm.Vt + 16 * tv0 * LDC, LDC);
            mma_nt_blk<WB::BR, C>(accC[pb], sm.Qtw + 16 * ti0 * LDC, LDC, sm.Vt + 16 * tv0 * LDC, LDC);
        });
        for (int i = threadIdx.x; i < D; i += NT) {
            sm.u0[i] = gc2 * sm.u0[i] + row_sum<T, C>(sm.Ztw, LDC, i);
            sm.m0[i] = gc * sm.m0[i] + row_sum<T, C>(sm.Qtw, LDC, i);
        }
        c0 = n0;
        cv = ncv;
    }
    __syncthreads();

    // summary [X = S | Y = C | N = W | y = m | nv = u]
    float *e = p.ws + ws_elem(bh, 0, p.spad, seg, G::SUMF);
    for_owned<SB, NW>(w, [&](int pb, int x, int y, int ti, int tj) {
#pragma unroll
        for (int i = 0; i < 4; ++i) e[(16 * ti + g4 + i) * D + 16 * tj + col] = accS[pb][x][y][i];
    });
    for_owned<WB, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = (16 * ti + g4 + i) * DV + 16 * tv + col;
            e[D * D + idx] = accC[pb][x][y][i];
            e[D * D + D * DV + idx] = accW[pb][x][y][i];
        }
    });
    for (int i = threadIdx.x; i < D; i += NT) {
        e[D * D + 2 * D * DV + i] = sm.m0[i];
        e[D * D + 2 * D * DV + D + i] = sm.u0[i];
    }
}

}  // namespace hla
