// ahla_kernels.h -- chunked asymmetric HLA (AHLA) on gfx950: segment-summary
// kernel and forward kernel.
//
// Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
// gist.science/es/paper/2510.27258, section "2. Atencion Lineal de Orden
// Superior Asimetrica (AHLA)": the operator Q (K^T Q)(K^T V), masked, with the
// streaming summaries P^KV, m^K, E and n.
//
// Chunk form (derived from those summaries): y_t = P_t^T q_t is causal linear
// attention, and o_t = q_t^T E_t with E_t = E_{t-1} + k_t y_t^T.  For a chunk
// with carried (P0, E0, mK0, nk0) and L = tril(Q K^T):
//     Y  = Q P0 + L V              y1 = Q mK0 + L 1      (v == 1 column)
//     O  = Q E0 + L Y              den = Q nk0 + L y1    (ratio form)
//     P0 += K^T V ; E0 += K^T Y ; mK0 += K^T 1 ; nk0 += K^T y1
// The summary kernel runs this from zero over one segment and also forms
// M = sum_t k_t q_t^T, the factor the segment combine's cross term M_B P_A
// needs.
//
// Work split as for HLA-2: wave (r, cg) owns row tile r and column tiles cg,
// cg + NCG, ...  The transposed scores L^T = K Q^T serve twice from
// registers: as the A operand of L V (rows tau) and as the B operand of
// Y^T L^T (for O^T).  Y is written to LDS transposed (for Y^T L^T and
// K^T Y), O^T goes straight to global memory.
#pragma once

#include "chunk_common.h"
#include "hla2_kernels.h"

namespace hla {

template <typename T, int D, int DV, int C>
struct AhlaCfg {
    using WS = WaveShape<C, D>;
    static constexpr int RT = WS::RT, NCG = WS::NCG, NW = WS::NW, NT = WS::NT;
    static constexpr int LDD = ld_of<T>(D), LDC = ld_of<T>(C);
    static constexpr int nTD = D / 16, nTV = DV / 16;
    static constexpr int OJ = (nTV + NCG - 1) / NCG;      // Y / O^T tiles per wave
    using PBk = TileBlocks<nTD, nTV, NW>;   // ownership of P, E tiles
    using MBk = TileBlocks<nTD, nTD, NW>;   // ownership of M tiles
    static constexpr int SUMF = summary_floats(D, DV);
    static constexpr int STF = ahla_state_floats(D, DV);
};

template <typename T, int D, int DV, int C>
struct AhlaFwdSmem {
    using G = AhlaCfg<T, D, DV, C>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T K[C * G::LDD];
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T Yt[DV * G::LDC];
    alignas(16) T Pt[DV * G::LDD];     // Pt[j][i] = P0[i][j]
    alignas(16) T Et[DV * G::LDD];     // Et[j][i] = E0[i][j]
    float mK[D], nk[D], y1[C];
};

template <typename T, int D, int DV, int C>
struct AhlaSumSmem {
    using G = AhlaCfg<T, D, DV, C>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T Qt[D * G::LDC];
    alignas(16) T K[C * G::LDD];
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T Yt[DV * G::LDC];
    alignas(16) T Pt[DV * G::LDD];
    float mK[D], nk[D], y1[C];
};

// Y = Q P0 + L V for row tile r (rows tau), written to Yt transposed; also
// y1[tau] = q_tau . mK + sum_sigma L[tau][sigma].
template <typename T, int D, int DV, int C, int RT, int NCG, int OJ, int LDD, int LDC>
__device__ __forceinline__ void ahla_y_phase(const Frag16<T> (&Lf)[RT], const RowFrags<T, D> &qf,
                                             int r, int cg, int tau, const T *Q, const T *Pt,
                                             const T *Vt, T *Yt, const float *mK, float *y1) {
    constexpr int nTV = DV / 16;
    const int g4 = (lane_id() >> 4) << 2;
#pragma unroll
    for (int jj = 0; jj < OJ; ++jj) {
        const int jv = cg + jj * NCG;
        if (jv < nTV) {
            // accumulator rows are tokens 16r + 4g + i, columns features 16 jv + c
            f32x4 y = mma_nt_fa(zero4(), qf, Pt + 16 * jv * LDD, LDD);
            f32x4 yc = zero4();
#pragma unroll
            for (int s = 0; s < RT; ++s)
                if (s <= r) yc = mma16(yc, Lf[s], ld_frag(Vt + 16 * jv * LDC + 16 * s, LDC));
            y += yc;
            store4(Yt + (16 * jv + acc_col()) * LDC + 16 * r + g4, y);
        }
    }
    if (cg == 0) {
        float rs = 0.f;
#pragma unroll
        for (int s = 0; s < RT; ++s)
            if (s <= r) {
#pragma unroll
                for (int i = 0; i < 4; ++i) rs += frag_val(Lf[s], i);
            }
        const float yv = lane_dot<T, D>(Q + tau * LDD, mK) + sum_groups(rs);
        if (lane_id() < 16) y1[tau] = yv;
    }
}

template <typename T, int D, int DV, int C>
__global__ __launch_bounds__((AhlaCfg<T, D, DV, C>::NT),
                             (hla2_min_blocks<AhlaCfg<T, D, DV, C>::NT, 0, D, DV>()))
void ahla_forward_kernel(FwdParams p) {
    using G = AhlaCfg<T, D, DV, C>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    constexpr int LDD = G::LDD, LDC = G::LDC, nTV = G::nTV;
    __shared__ AhlaFwdSmem<T, D, DV, C> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
    const int r = w / NCG, cg = w % NCG;
    const int col = acc_col(), g = lane_id() >> 4, g4 = g << 2;
    const int tau = 16 * r + col;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * p.n * DV;

    const float *P0 = nullptr, *E0 = nullptr, *mK0 = nullptr, *nk0 = nullptr;
    if (p.nseg > 1) {
        const float *e = p.ws + ws_elem(bh, 1, p.spad, seg, G::SUMF);
        P0 = e + D * D;
        E0 = e + D * D + D * DV;
        mK0 = e + D * D + 2 * D * DV;
        nk0 = mK0 + D;
    } else if (p.state_in) {
        const float *e = p.state_in + (size_t)bh * G::STF;
        P0 = e;
        E0 = e + D * DV;
        mK0 = e + 2 * D * DV;
        nk0 = mK0 + D;
    }
    using PBk = typename G::PBk;
    f32x4 accP[PBk::PB][PBk::BR][PBk::BR], accE[PBk::PB][PBk::BR][PBk::BR];
    for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
        f32x4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = (16 * ti + g4 + i) * DV + 16 * tv + col;
            a[i] = P0 ? P0[idx] : 0.f;
            b[i] = E0 ? E0[idx] : 0.f;
        }
        accP[pb][x][y] = a;
        accE[pb][x][y] = b;
        store4(sm.Pt + (16 * tv + col) * LDD + 16 * ti + g4, a);
        store4(sm.Et + (16 * tv + col) * LDD + 16 * ti + g4, b);
    });
    for (int i = threadIdx.x; i < D; i += NT) {
        sm.mK[i] = mK0 ? mK0[i] : 0.f;
        sm.nk[i] = nk0 ? nk0[i] : 0.f;
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
        rk.store_rows(sm.K, LDD);
        rk.store_cols(sm.Kt, LDC);
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
        scores_t<T, D, RT, LDD, false>(Lf, sm.K, qf, r, tau, nullptr, 1);
        ahla_y_phase<T, D, DV, C, RT, NCG, G::OJ, LDD, LDC>(Lf, qf, r, cg, tau, sm.Q, sm.Pt, sm.Vt,
                                                            sm.Yt, sm.mK, sm.y1);
        // carried part of the output and of its denominator
        f32x4 accO[G::OJ];
#pragma unroll
        for (int jj = 0; jj < G::OJ; ++jj) {
            const int jv = cg + jj * NCG;
            accO[jj] = zero4();
            if (jv < nTV) accO[jj] = mma_nt_f(zero4(), sm.Et + 16 * jv * LDD, LDD, qf);
        }
        float den = 0.f;
        if (p.ratio) den = lane_dot<T, D>(sm.Q + tau * LDD, sm.nk);
        __syncthreads();

        // O^T += Y^T L^T ; den += sum_sigma L[tau][sigma] y1[sigma]
        if (p.ratio) {
            float a = 0.f;
#pragma unroll
            for (int s = 0; s < RT; ++s)
                if (s <= r) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) a += frag_val(Lf[s], i) * sm.y1[16 * s + g4 + i];
                }
            den += sum_groups(a);
        }
#pragma unroll
        for (int jj = 0; jj < G::OJ; ++jj) {
            const int jv = cg + jj * NCG;
            if (jv < nTV) {
                f32x4 oc = zero4();
#pragma unroll
                for (int s = 0; s < RT; ++s)
                    if (s <= r) oc = mma16(oc, ld_frag(sm.Yt + 16 * jv * LDC + 16 * s, LDC), Lf[s]);
                f32x4 ov = accO[jj] + oc;
                if (p.ratio) ov *= 1.f / den;
                if (tau < cv) store4(o + (size_t)(c0 + tau) * DV + 16 * jv + g4, ov);
            }
        }
        // advance the state: P0 += K^T V, E0 += K^T Y, mK0 += K^T 1, nk0 += K^T y1
        for_blocks<PBk, NW>(w, [&](int pb, int ti0, int tv0) {
            mma_nt_blk<PBk::BR, C>(accP[pb], sm.Kt + 16 * ti0 * LDC, LDC, sm.Vt + 16 * tv0 * LDC, LDC);
            mma_nt_blk<PBk::BR, C>(accE[pb], sm.Kt + 16 * ti0 * LDC, LDC, sm.Yt + 16 * tv0 * LDC, LDC);
#pragma unroll
            for (int x = 0; x < PBk::BR; ++x)
#pragma unroll
                for (int y = 0; y < PBk::BR; ++y) {
                    const int o = (16 * (tv0 + y) + col) * LDD + 16 * (ti0 + x) + g4;
                    store4(sm.Pt + o, accP[pb][x][y]);
                    store4(sm.Et + o, accE[pb][x][y]);
                }
        });
        for (int i = threadIdx.x; i < D; i += NT) {
            sm.mK[i] += row_sum<T, C>(sm.Kt, LDC, i);
            sm.nk[i] += row_dot<T, C>(sm.Kt, LDC, i, sm.y1);
        }
        c0 = n0;
        cv = ncv;
    }

    if (p.state_out && seg == p.nseg - 1) {
        float *so = p.state_out + (size_t)bh * G::STF;
        for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = (16 * ti + g4 + i) * DV + 16 * tv + col;
                so[idx] = accP[pb][x][y][i];
                so[D * DV + idx] = accE[pb][x][y][i];
            }
        });
        __syncthreads();
        for (int i = threadIdx.x; i < D; i += NT) {
            so[2 * D * DV + i] = sm.mK[i];
            so[2 * D * DV + D + i] = sm.nk[i];
        }
    }
}

template <typename T, int D, int DV, int C>
__global__ __launch_bounds__((AhlaCfg<T, D, DV, C>::NT),
                             (hla2_min_blocks<AhlaCfg<T, D, DV, C>::NT, 0, D, DV>()))
void ahla_summary_kernel(FwdParams p) {
    using G = AhlaCfg<T, D, DV, C>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    constexpr int LDD = G::LDD, LDC = G::LDC, nTD = G::nTD, nTV = G::nTV;
    __shared__ AhlaSumSmem<T, D, DV, C> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
    const int r = w / NCG, cg = w % NCG;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const int tau = 16 * r + col;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;

    using PBk = typename G::PBk;
    using MBk = typename G::MBk;
    f32x4 accP[PBk::PB][PBk::BR][PBk::BR], accE[PBk::PB][PBk::BR][PBk::BR];
    f32x4 accM[MBk::PB][MBk::BR][MBk::BR];
#pragma unroll
    for (int pb = 0; pb < PBk::PB; ++pb)
#pragma unroll
        for (int x = 0; x < PBk::BR; ++x)
#pragma unroll
            for (int y = 0; y < PBk::BR; ++y) {
                accP[pb][x][y] = zero4();
                accE[pb][x][y] = zero4();
            }
#pragma unroll
    for (int pb = 0; pb < MBk::PB; ++pb)
#pragma unroll
        for (int x = 0; x < MBk::BR; ++x)
#pragma unroll
            for (int y = 0; y < MBk::BR; ++y) accM[pb][x][y] = zero4();
    for (int i = threadIdx.x; i < DV * LDD; i += NT) sm.Pt[i] = from_f<T>(0.f);
    for (int i = threadIdx.x; i < D; i += NT) {
        sm.mK[i] = 0.f;
        sm.nk[i] = 0.f;
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
        rq.store_cols(sm.Qt, LDC);
        rk.store_rows(sm.K, LDD);
        rk.store_cols(sm.Kt, LDC);
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
        scores_t<T, D, RT, LDD, false>(Lf, sm.K, qf, r, tau, nullptr, 1);
        ahla_y_phase<T, D, DV, C, RT, NCG, G::OJ, LDD, LDC>(Lf, qf, r, cg, tau, sm.Q, sm.Pt, sm.Vt,
                                                            sm.Yt, sm.mK, sm.y1);
        __syncthreads();

        for_blocks<PBk, NW>(w, [&](int pb, int ti0, int tv0) {
            mma_nt_blk<PBk::BR, C>(accP[pb], sm.Kt + 16 * ti0 * LDC, LDC, sm.Vt + 16 * tv0 * LDC, LDC);
            mma_nt_blk<PBk::BR, C>(accE[pb], sm.Kt + 16 * ti0 * LDC, LDC, sm.Yt + 16 * tv0 * LDC, LDC);
#pragma unroll
            for (int x = 0; x < PBk::BR; ++x)
#pragma unroll
                for (int y = 0; y < PBk::BR; ++y)
                    store4(sm.Pt + (16 * (tv0 + y) + col) * LDD + 16 * (ti0 + x) + g4, accP[pb][x][y]);
        });
        for_blocks<MBk, NW>(w, [&](int pb, int ti0, int tj0) {
            mma_nt_blk<MBk::BR, C>(accM[pb], sm.Kt + 16 * ti0 * LDC, LDC, sm.Qt + 16 * tj0 * LDC, LDC);
        });
        for (int i = threadIdx.x; i < D; i += NT) {
            sm.mK[i] += row_sum<T, C>(sm.Kt, LDC, i);
            sm.nk[i] += row_dot<T, C>(sm.Kt, LDC, i, sm.y1);
        }
        c0 = n0;
        cv = ncv;
    }
    __syncthreads();

    // summary [X = M | Y = P | N = E | y = mK | nv = nk]
    float *e = p.ws + ws_elem(bh, 0, p.spad, seg, G::SUMF);
    for_owned<MBk, NW>(w, [&](int pb, int x, int y, int ti, int tj) {
#pragma unroll
        for (int i = 0; i < 4; ++i) e[(16 * ti + g4 + i) * D + 16 * tj + col] = accM[pb][x][y][i];
    });
    for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = (16 * ti + g4 + i) * DV + 16 * tv + col;
            e[D * D + idx] = accP[pb][x][y][i];
            e[D * D + D * DV + idx] = accE[pb][x][y][i];
        }
    });
    for (int i = threadIdx.x; i < D; i += NT) {
        e[D * D + 2 * D * DV + i] = sm.mK[i];
        e[D * D + 2 * D * DV + D + i] = sm.nk[i];
    }
}

}  // namespace hla
