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
#pragma once

#include "device_common.h"
#include "hla2_kernels.h"
#include "params.h"

namespace hla {

template <typename T, int D, int DV, int C, int NW>
struct AhlaCfg {
    static constexpr int NT = NW * kWave;
    static constexpr int LDD = ld_of<T>(D), LDC = ld_of<T>(C), LDV = ld_of<T>(DV);
    static constexpr int nTC = C / 16, nTD = D / 16, nTV = DV / 16;
    static constexpr int TY = nTC * nTV;                 // C x DV tiles (Y, O)
    static constexpr int TP = nTD * nTV;                 // D x DV tiles (P, E)
    static constexpr int TM = nTD * nTD;                 // D x D tiles (M)
    static constexpr int PY = (TY + NW - 1) / NW, PP = (TP + NW - 1) / NW, PM = (TM + NW - 1) / NW;
    static constexpr int SUMF = summary_floats(D, DV);
    static constexpr int STF = ahla_state_floats(D, DV);
    static constexpr int KO = (C * LDD > C * LDV) ? C * LDD : C * LDV;
};

template <typename T, int D, int DV, int C, int NW>
struct AhlaFwdSmem {
    using G = AhlaCfg<T, D, DV, C, NW>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T K[G::KO];            // K rows (scores), later output staging
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T L[C * G::LDC];
    alignas(16) T Yt[DV * G::LDC];
    alignas(16) T Pt[DV * G::LDD];     // Pt[j][i] = P0[i][j]
    alignas(16) T Et[DV * G::LDD];     // Et[j][i] = E0[i][j]
    float mK[D], nk[D], y1[C], den[C];
};

template <typename T, int D, int DV, int C, int NW>
struct AhlaSumSmem {
    using G = AhlaCfg<T, D, DV, C, NW>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T Qt[D * G::LDC];
    alignas(16) T K[C * G::LDD];
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T L[C * G::LDC];
    alignas(16) T Yt[DV * G::LDC];
    alignas(16) T Pt[DV * G::LDD];
    float mK[D], nk[D], y1[C];
};

template <typename T, int D, int DV, int C, int NW>
__global__ __launch_bounds__(NW * kWave) void ahla_forward_kernel(FwdParams p) {
    using G = AhlaCfg<T, D, DV, C, NW>;
    constexpr int NT = G::NT, LDD = G::LDD, LDC = G::LDC, LDV = G::LDV;
    constexpr int nTV = G::nTV;
    __shared__ AhlaFwdSmem<T, D, DV, C, NW> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
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
    f32x4 accP[G::PP], accE[G::PP];
#pragma unroll
    for (int s = 0; s < G::PP; ++s) {
        const int t = w + s * NW;
        accP[s] = zero4();
        accE[s] = zero4();
        if (t < G::TP) {
            const int ti = t / nTV, tj = t % nTV;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                const float xp = P0 ? P0[row * DV + col] : 0.f;
                const float xe = E0 ? E0[row * DV + col] : 0.f;
                accP[s][r] = xp;
                accE[s][r] = xe;
                sm.Pt[col * LDD + row] = from_f<T>(xp);
                sm.Et[col * LDD + row] = from_f<T>(xe);
            }
        }
    }
    for (int i = threadIdx.x; i < D; i += NT) {
        sm.mK[i] = mK0 ? mK0[i] : 0.f;
        sm.nk[i] = nk0 ? nk0[i] : 0.f;
    }

    for (int c0 = t_begin; c0 < t_end; c0 += C) {
        const int cv = min(C, t_end - c0);
        __syncthreads();
        stage_tile<T, C, D, NT>(q + (size_t)c0 * D, cv, sm.Q, LDD, nullptr, 0);
        stage_tile<T, C, D, NT>(k + (size_t)c0 * D, cv, sm.K, LDD, sm.Kt, LDC);
        stage_tile<T, C, DV, NT>(v + (size_t)c0 * DV, cv, nullptr, 0, sm.Vt, LDC);
        __syncthreads();

        // scores and carried-state terms Q P0, Q E0, Q mK0, Q nk0
        scores_tril<T, D, C, false, NW, LDD, LDC>(sm.Q, sm.K, sm.L, nullptr);
        f32x4 accY[G::PY], accO[G::PY];
#pragma unroll
        for (int s = 0; s < G::PY; ++s) {
            const int t = w + s * NW;
            accY[s] = zero4();
            accO[s] = zero4();
            if (t < G::TY) {
                const int ti = t / nTV, tj = t % nTV;
                accY[s] = mma_nt(accY[s], sm.Q + ti * 16 * LDD, LDD, sm.Pt + tj * 16 * LDD, LDD, 0, D);
                accO[s] = mma_nt(accO[s], sm.Q + ti * 16 * LDD, LDD, sm.Et + tj * 16 * LDD, LDD, 0, D);
            }
        }
        for (int i = threadIdx.x; i < C; i += NT) {
            float a = 0.f, b = 0.f;
            for (int c = 0; c < D; ++c) {
                const float x = to_f(sm.Q[i * LDD + c]);
                a += x * sm.mK[c];
                b += x * sm.nk[c];
            }
            sm.y1[i] = a;
            sm.den[i] = b;
        }
        __syncthreads();

        // Y = Q P0 + L V ; P0 += K^T V ; y1 += L 1
#pragma unroll
        for (int s = 0; s < G::PY; ++s) {
            const int t = w + s * NW;
            if (t < G::TY) {
                const int ti = t / nTV, tj = t % nTV;
                accY[s] = mma_nt(accY[s], sm.L + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0,
                                 (ti + 1) * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.Yt[(tj * 16 + acc_col()) * LDC + ti * 16 + acc_row(r)] = from_f<T>(accY[s][r]);
            }
        }
#pragma unroll
        for (int s = 0; s < G::PP; ++s) {
            const int t = w + s * NW;
            if (t < G::TP) {
                const int ti = t / nTV, tj = t % nTV;
                accP[s] = mma_nt(accP[s], sm.Kt + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0, C);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.Pt[(tj * 16 + acc_col()) * LDD + ti * 16 + acc_row(r)] = from_f<T>(accP[s][r]);
            }
        }
        for (int i = threadIdx.x; i < C; i += NT) {
            float a = 0.f;
            for (int c = 0; c <= i; ++c) a += to_f(sm.L[i * LDC + c]);
            sm.y1[i] += a;
        }
        __syncthreads();

        // O = Q E0 + L Y ; E0 += K^T Y ; den += L y1 ; nk += K^T y1 ; mK += K^T 1
#pragma unroll
        for (int s = 0; s < G::PY; ++s) {
            const int t = w + s * NW;
            if (t < G::TY) {
                const int ti = t / nTV, tj = t % nTV;
                accO[s] = mma_nt(accO[s], sm.L + ti * 16 * LDC, LDC, sm.Yt + tj * 16 * LDC, LDC, 0,
                                 (ti + 1) * 16);
            }
        }
#pragma unroll
        for (int s = 0; s < G::PP; ++s) {
            const int t = w + s * NW;
            if (t < G::TP) {
                const int ti = t / nTV, tj = t % nTV;
                accE[s] = mma_nt(accE[s], sm.Kt + ti * 16 * LDC, LDC, sm.Yt + tj * 16 * LDC, LDC, 0, C);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.Et[(tj * 16 + acc_col()) * LDD + ti * 16 + acc_row(r)] = from_f<T>(accE[s][r]);
            }
        }
        for (int i = threadIdx.x; i < C; i += NT) {
            float a = 0.f;
            for (int c = 0; c <= i; ++c) a += to_f(sm.L[i * LDC + c]) * sm.y1[c];
            sm.den[i] += a;
        }
        for (int i = threadIdx.x; i < D; i += NT) {
            float a = 0.f, b = 0.f;
            for (int c = 0; c < C; ++c) {
                const float x = to_f(sm.Kt[i * LDC + c]);
                a += x;
                b += x * sm.y1[c];
            }
            sm.mK[i] += a;
            sm.nk[i] += b;
        }
        __syncthreads();

        T *Os = sm.K;
#pragma unroll
        for (int s = 0; s < G::PY; ++s) {
            const int t = w + s * NW;
            if (t < G::TY) {
                const int ti = t / nTV, tj = t % nTV;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                    float ov = accO[s][r];
                    if (p.ratio) ov = ov / sm.den[row];
                    Os[row * LDV + col] = from_f<T>(ov);
                }
            }
        }
        __syncthreads();
        {
            constexpr int VE = Vec16<T>::N;
            constexpr int VPR = DV / VE;
            for (int idx = threadIdx.x; idx < cv * VPR; idx += NT) {
                const int r = idx / VPR, c = (idx % VPR) * VE;
                store16(o + (size_t)(c0 + r) * DV + c, load16(Os + r * LDV + c));
            }
        }
    }

    if (p.state_out && seg == p.nseg - 1) {
        float *so = p.state_out + (size_t)bh * G::STF;
#pragma unroll
        for (int s = 0; s < G::PP; ++s) {
            const int t = w + s * NW;
            if (t < G::TP) {
                const int ti = t / nTV, tj = t % nTV;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int idx = (ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col();
                    so[idx] = accP[s][r];
                    so[D * DV + idx] = accE[s][r];
                }
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < D; i += NT) {
            so[2 * D * DV + i] = sm.mK[i];
            so[2 * D * DV + D + i] = sm.nk[i];
        }
    }
}

template <typename T, int D, int DV, int C, int NW>
__global__ __launch_bounds__(NW * kWave) void ahla_summary_kernel(FwdParams p) {
    using G = AhlaCfg<T, D, DV, C, NW>;
    constexpr int NT = G::NT, LDD = G::LDD, LDC = G::LDC;
    constexpr int nTD = G::nTD, nTV = G::nTV;
    __shared__ AhlaSumSmem<T, D, DV, C, NW> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;

    f32x4 accP[G::PP], accE[G::PP], accM[G::PM];
#pragma unroll
    for (int s = 0; s < G::PP; ++s) { accP[s] = zero4(); accE[s] = zero4(); }
#pragma unroll
    for (int s = 0; s < G::PM; ++s) accM[s] = zero4();
    for (int i = threadIdx.x; i < DV * LDD; i += NT) sm.Pt[i] = from_f<T>(0.f);
    for (int i = threadIdx.x; i < D; i += NT) { sm.mK[i] = 0.f; sm.nk[i] = 0.f; }

    for (int c0 = t_begin; c0 < t_end; c0 += C) {
        const int cv = min(C, t_end - c0);
        __syncthreads();
        stage_tile<T, C, D, NT>(q + (size_t)c0 * D, cv, sm.Q, LDD, sm.Qt, LDC);
        stage_tile<T, C, D, NT>(k + (size_t)c0 * D, cv, sm.K, LDD, sm.Kt, LDC);
        stage_tile<T, C, DV, NT>(v + (size_t)c0 * DV, cv, nullptr, 0, sm.Vt, LDC);
        __syncthreads();

        scores_tril<T, D, C, false, NW, LDD, LDC>(sm.Q, sm.K, sm.L, nullptr);
        f32x4 accY[G::PY];
#pragma unroll
        for (int s = 0; s < G::PY; ++s) {
            const int t = w + s * NW;
            accY[s] = zero4();
            if (t < G::TY) {
                const int ti = t / nTV, tj = t % nTV;
                accY[s] = mma_nt(accY[s], sm.Q + ti * 16 * LDD, LDD, sm.Pt + tj * 16 * LDD, LDD, 0, D);
            }
        }
        for (int i = threadIdx.x; i < C; i += NT) {
            float a = 0.f;
            for (int c = 0; c < D; ++c) a += to_f(sm.Q[i * LDD + c]) * sm.mK[c];
            sm.y1[i] = a;
        }
        __syncthreads();

#pragma unroll
        for (int s = 0; s < G::PY; ++s) {
            const int t = w + s * NW;
            if (t < G::TY) {
                const int ti = t / nTV, tj = t % nTV;
                accY[s] = mma_nt(accY[s], sm.L + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0,
                                 (ti + 1) * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.Yt[(tj * 16 + acc_col()) * LDC + ti * 16 + acc_row(r)] = from_f<T>(accY[s][r]);
            }
        }
#pragma unroll
        for (int s = 0; s < G::PP; ++s) {
            const int t = w + s * NW;
            if (t < G::TP) {
                const int ti = t / nTV, tj = t % nTV;
                accP[s] = mma_nt(accP[s], sm.Kt + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0, C);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.Pt[(tj * 16 + acc_col()) * LDD + ti * 16 + acc_row(r)] = from_f<T>(accP[s][r]);
            }
        }
        for (int i = threadIdx.x; i < C; i += NT) {
            float a = 0.f;
            for (int c = 0; c <= i; ++c) a += to_f(sm.L[i * LDC + c]);
            sm.y1[i] += a;
        }
        __syncthreads();

#pragma unroll
        for (int s = 0; s < G::PP; ++s) {
            const int t = w + s * NW;
            if (t < G::TP) {
                const int ti = t / nTV, tj = t % nTV;
                accE[s] = mma_nt(accE[s], sm.Kt + ti * 16 * LDC, LDC, sm.Yt + tj * 16 * LDC, LDC, 0, C);
            }
        }
#pragma unroll
        for (int s = 0; s < G::PM; ++s) {
            const int t = w + s * NW;
            if (t < G::TM) {
                const int ti = t / nTD, tj = t % nTD;
                accM[s] = mma_nt(accM[s], sm.Kt + ti * 16 * LDC, LDC, sm.Qt + tj * 16 * LDC, LDC, 0, C);
            }
        }
        for (int i = threadIdx.x; i < D; i += NT) {
            float a = 0.f, b = 0.f;
            for (int c = 0; c < C; ++c) {
                const float x = to_f(sm.Kt[i * LDC + c]);
                a += x;
                b += x * sm.y1[c];
            }
            sm.mK[i] += a;
            sm.nk[i] += b;
        }
    }
    __syncthreads();

    // summary [X = M | Y = P | N = E | y = mK | nv = nk]
    float *e = p.ws + ws_elem(bh, 0, p.spad, seg, G::SUMF);
#pragma unroll
    for (int s = 0; s < G::PM; ++s) {
        const int t = w + s * NW;
        if (t < G::TM) {
            const int ti = t / nTD, tj = t % nTD;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                e[(ti * 16 + acc_row(r)) * D + tj * 16 + acc_col()] = accM[s][r];
        }
    }
#pragma unroll
    for (int s = 0; s < G::PP; ++s) {
        const int t = w + s * NW;
        if (t < G::TP) {
            const int ti = t / nTV, tj = t % nTV;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = (ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col();
                e[D * D + idx] = accP[s][r];
                e[D * D + D * DV + idx] = accE[s][r];
            }
        }
    }
    for (int i = threadIdx.x; i < D; i += NT) {
        e[D * D + 2 * D * DV + i] = sm.mK[i];
        e[D * D + 2 * D * DV + D + i] = sm.nk[i];
    }
}

}  // namespace hla
