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
// Work split: NW waves; every product is a set of 16x16 MFMA tiles dealt
// round-robin to the waves.  The fp32 state S0, W0 lives in MFMA accumulators
// for the whole segment; its T-typed copy (transposed, the Bt operand of
// Q S0 and Q W0) is refreshed in LDS once per chunk.
#pragma once

#include "device_common.h"
#include "params.h"

namespace hla {

template <typename T, int D, int DV, int C, bool DECAY, int NW>
struct Hla2Cfg {
    static constexpr int NT = NW * kWave;
    static constexpr int LDD = ld_of<T>(D);   // rows of length D
    static constexpr int LDC = ld_of<T>(C);   // rows of length C
    static constexpr int LDV = ld_of<T>(DV);  // rows of length DV
    static constexpr int nTC = C / 16, nTD = D / 16, nTV = DV / 16;
    static constexpr int TZ = nTC * nTD, TO = nTC * nTV, TS = nTD * nTD, TW = nTD * nTV;
    static constexpr int TL = nTC * (nTC + 1) / 2;       // lower-triangular chunk tiles
    static constexpr int PZ = (TZ + NW - 1) / NW, PO = (TO + NW - 1) / NW;
    static constexpr int PS = (TS + NW - 1) / NW, PW = (TW + NW - 1) / NW;
    static constexpr int SUMF = summary_floats(D, DV);
    static constexpr int STF = hla2_state_floats(D, DV);
    static constexpr int KO = (C * LDD > C * LDV) ? C * LDD : C * LDV;  // K rows / output staging
    static constexpr int NPOW = 2 * C + 2;
    static_assert(D % 16 == 0 && DV % 16 == 0 && C % 16 == 0, "tile multiples");
};

template <typename T, int D, int DV, int C, bool DECAY, int NW>
struct Hla2FwdSmem {
    using G = Hla2Cfg<T, D, DV, C, DECAY, NW>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T K[G::KO];            // K rows in stage 1, output staging in stage 4
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Ktw[DECAY ? D * G::LDC : 8];
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T L[C * G::LDC];
    alignas(16) T Z[C * G::LDD];
    alignas(16) T Ztw[D * G::LDC];
    alignas(16) T P[C * G::LDC];
    alignas(16) T St[D * G::LDD];      // St[j][i] = S0[i][j]
    alignas(16) T Wt[DV * G::LDD];     // Wt[j][i] = W0[i][j]
    float u[D];
    float den[C];                      // carried-state part of the denominator
    float denp[C][G::nTC];             // row sums of P, one per 16-column tile
    float gp[G::NPOW];
};

template <typename T, int D, int DV, int C, bool DECAY, int NW>
struct Hla2SumSmem {
    using G = Hla2Cfg<T, D, DV, C, DECAY, NW>;
    alignas(16) T Q[C * G::LDD];
    alignas(16) T Qtw[D * G::LDC];     // Q^T weighted by g^(c-1-tau)
    alignas(16) T K[C * G::LDD];
    alignas(16) T Kt[D * G::LDC];
    alignas(16) T Ktw[DECAY ? D * G::LDC : 8];
    alignas(16) T Vt[DV * G::LDC];
    alignas(16) T L[C * G::LDC];
    alignas(16) T Ztw[D * G::LDC];
    alignas(16) T St[D * G::LDD];
    float u[D];
    float m[D];
    float gp[G::NPOW];
};

// ---------------------------------------------------------------- helpers

// scores L = D_g * tril(Q K^T) into LDS (lower tiles only; upper tiles of L
// are never read because every consumer stops its k loop at the diagonal)
template <typename T, int D, int C, bool DECAY, int NW, int LDD, int LDC>
__device__ __forceinline__ void scores_tril(const T *Q, const T *K, T *L, const float *gp) {
    constexpr int nTC = C / 16;
    const int w = wave_id();
    int t = 0;
    for (int ti = 0; ti < nTC; ++ti) {
        for (int tj = 0; tj <= ti; ++tj, ++t) {
            if (t % NW != w) continue;
            f32x4 a = mma_nt(zero4(), Q + ti * 16 * LDD, LDD, K + tj * 16 * LDD, LDD, 0, D);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                float val = 0.f;
                if (col <= row) val = DECAY ? a[r] * gp[row - col] : a[r];
                L[row * LDC + col] = from_f<T>(val);
            }
        }
    }
}

// ------------------------------------------------------------ forward kernel

template <typename T, int D, int DV, int C, bool DECAY, int NW>
__global__ __launch_bounds__(NW * kWave) void hla2_forward_kernel(FwdParams p) {
    using G = Hla2Cfg<T, D, DV, C, DECAY, NW>;
    constexpr int NT = G::NT, LDD = G::LDD, LDC = G::LDC, LDV = G::LDV;
    constexpr int nTC = G::nTC, nTD = G::nTD, nTV = G::nTV;
    __shared__ Hla2FwdSmem<T, D, DV, C, DECAY, NW> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
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
    f32x4 accS[G::PS], accW[G::PW];
#pragma unroll
    for (int s = 0; s < G::PS; ++s) {
        const int t = w + s * NW;
        accS[s] = zero4();
        if (t < G::TS) {
            const int ti = t / nTD, tj = t % nTD;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                const float x = S0 ? S0[row * D + col] : 0.f;
                accS[s][r] = x;
                sm.St[col * LDD + row] = from_f<T>(x);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < G::PW; ++s) {
        const int t = w + s * NW;
        accW[s] = zero4();
        if (t < G::TW) {
            const int ti = t / nTV, tj = t % nTV;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                const float x = W0 ? W0[row * DV + col] : 0.f;
                accW[s][r] = x;
                sm.Wt[col * LDD + row] = from_f<T>(x);
            }
        }
    }
    for (int i = threadIdx.x; i < D; i += NT) sm.u[i] = u0 ? u0[i] : 0.f;

    for (int c0 = t_begin; c0 < t_end; c0 += C) {
        const int cv = min(C, t_end - c0);
        __syncthreads();  // previous chunk's output staging has been stored; gp ready
        // ---- a-1: stage Q, K (row-major, transposed, decay-weighted) and V^T
        stage_tile<T, C, D, NT>(q + (size_t)c0 * D, cv, sm.Q, LDD, nullptr, 0);
        if (DECAY) {
            // weights g^(cv-1-tau) for the S0 update
            const int VE = Vec16<T>::N;
            for (int idx = threadIdx.x; idx < C * (D / VE); idx += NT) {
                const int r = idx / (D / VE), c = (idx % (D / VE)) * VE;
                Vec16<T> x;
                if (r < cv) x = load16(k + (size_t)(c0 + r) * D + c);
                else {
#pragma unroll
                    for (int e = 0; e < VE; ++e) x.v[e] = from_f<T>(0.f);
                }
                store16(sm.K + r * LDD + c, x);
                const float wr = (r < cv) ? sm.gp[cv - 1 - r] : 0.f;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    sm.Kt[(c + e) * LDC + r] = x.v[e];
                    sm.Ktw[(c + e) * LDC + r] = from_f<T>(to_f(x.v[e]) * wr);
                }
            }
        } else {
            stage_tile<T, C, D, NT>(k + (size_t)c0 * D, cv, sm.K, LDD, sm.Kt, LDC);
        }
        stage_tile<T, C, DV, NT>(v + (size_t)c0 * DV, cv, nullptr, 0, sm.Vt, LDC);
        __syncthreads();

        // ---- a-2: scores; a-3/a-4 carried-state terms Q S0, Q W0 (and Q u0)
        scores_tril<T, D, C, DECAY, NW, LDD, LDC>(sm.Q, sm.K, sm.L, sm.gp);
        f32x4 accZ[G::PZ], accO[G::PO];
#pragma unroll
        for (int s = 0; s < G::PZ; ++s) {
            const int t = w + s * NW;
            accZ[s] = zero4();
            if (t < G::TZ) {
                const int ti = t / nTD, tj = t % nTD;
                accZ[s] = mma_nt(accZ[s], sm.Q + ti * 16 * LDD, LDD, sm.St + tj * 16 * LDD, LDD, 0, D);
            }
        }
#pragma unroll
        for (int s = 0; s < G::PO; ++s) {
            const int t = w + s * NW;
            accO[s] = zero4();
            if (t < G::TO) {
                const int ti = t / nTV, tj = t % nTV;
                accO[s] = mma_nt(accO[s], sm.Q + ti * 16 * LDD, LDD, sm.Wt + tj * 16 * LDD, LDD, 0, D);
            }
        }
        if (p.ratio) {
            for (int i = threadIdx.x; i < C; i += NT) {
                float s = 0.f;
                for (int a = 0; a < D; ++a) s += to_f(sm.Q[i * LDD + a]) * sm.u[a];
                sm.den[i] = DECAY ? s * sm.gp[2 * (i + 1)] : s;
            }
        }
        __syncthreads();

        // ---- a-3: Z = diag(g^(tau+1)) Q S0 + L K
#pragma unroll
        for (int s = 0; s < G::PZ; ++s) {
            const int t = w + s * NW;
            if (t < G::TZ) {
                const int ti = t / nTD, tj = t % nTD;
                if (DECAY) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) accZ[s][r] *= sm.gp[ti * 16 + acc_row(r) + 1];
                }
                accZ[s] = mma_nt(accZ[s], sm.L + ti * 16 * LDC, LDC, sm.Kt + tj * 16 * LDC, LDC, 0,
                                 (ti + 1) * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                    const float z = accZ[s][r];
                    sm.Z[row * LDD + col] = from_f<T>(z);
                    float wz = 0.f;
                    if (row < cv) wz = DECAY ? sm.gp[2 * (cv - 1 - row)] : 1.f;
                    sm.Ztw[col * LDC + row] = from_f<T>(z * wz);
                }
            }
        }
        __syncthreads();

        // ---- a-4: P = D_{g^2} * tril(Q Z^T) (+ row sums for the ratio form)
        {
            int t = 0;
            for (int ti = 0; ti < nTC; ++ti) {
                for (int tj = 0; tj <= ti; ++tj, ++t) {
                    if (t % NW != w) continue;
                    f32x4 a = mma_nt(zero4(), sm.Q + ti * 16 * LDD, LDD, sm.Z + tj * 16 * LDD, LDD, 0, D);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                        float val = 0.f;
                        if (col <= row) val = DECAY ? a[r] * sm.gp[2 * (row - col)] : a[r];
                        const T tv = from_f<T>(val);
                        sm.P[row * LDC + col] = tv;
                        if (p.ratio) {
                            float rs = to_f(tv);
                            rs += __shfl_xor(rs, 1, 16);
                            rs += __shfl_xor(rs, 2, 16);
                            rs += __shfl_xor(rs, 4, 16);
                            rs += __shfl_xor(rs, 8, 16);
                            if (acc_col() == 0) sm.denp[row][tj] = rs;
                        }
                    }
                }
            }
        }
        // ---- a-7: advance the carried state by this chunk
        const float gc = DECAY ? sm.gp[cv] : 1.f;
        const float gc2 = DECAY ? sm.gp[2 * cv] : 1.f;
        const T *KA = DECAY ? sm.Ktw : sm.Kt;
#pragma unroll
        for (int s = 0; s < G::PS; ++s) {
            const int t = w + s * NW;
            if (t < G::TS) {
                const int ti = t / nTD, tj = t % nTD;
                if (DECAY) accS[s] *= gc;
                accS[s] = mma_nt(accS[s], KA + ti * 16 * LDC, LDC, sm.Kt + tj * 16 * LDC, LDC, 0, C);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.St[(tj * 16 + acc_col()) * LDD + ti * 16 + acc_row(r)] = from_f<T>(accS[s][r]);
            }
        }
#pragma unroll
        for (int s = 0; s < G::PW; ++s) {
            const int t = w + s * NW;
            if (t < G::TW) {
                const int ti = t / nTV, tj = t % nTV;
                if (DECAY) accW[s] *= gc2;
                accW[s] = mma_nt(accW[s], sm.Ztw + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0, C);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.Wt[(tj * 16 + acc_col()) * LDD + ti * 16 + acc_row(r)] = from_f<T>(accW[s][r]);
            }
        }
        for (int i = threadIdx.x; i < D; i += NT) {
            float s = 0.f;
            for (int c = 0; c < C; ++c) s += to_f(sm.Ztw[i * LDC + c]);
            sm.u[i] = gc2 * sm.u[i] + s;
        }
        __syncthreads();

        // ---- a-4: O = diag(g^(2(tau+1))) Q W0 + P V  (/ den)
        T *Os = sm.K;
#pragma unroll
        for (int s = 0; s < G::PO; ++s) {
            const int t = w + s * NW;
            if (t < G::TO) {
                const int ti = t / nTV, tj = t % nTV;
                if (DECAY) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) accO[s][r] *= sm.gp[2 * (ti * 16 + acc_row(r) + 1)];
                }
                accO[s] = mma_nt(accO[s], sm.P + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0,
                                 (ti + 1) * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                    float ov = accO[s][r];
                    if (p.ratio) {
                        float den = sm.den[row];
                        for (int c = 0; c <= ti; ++c) den += sm.denp[row][c];
                        ov = ov / den;
                    }
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
        for (int s = 0; s < G::PS; ++s) {
            const int t = w + s * NW;
            if (t < G::TS) {
                const int ti = t / nTD, tj = t % nTD;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    so[(ti * 16 + acc_row(r)) * D + tj * 16 + acc_col()] = accS[s][r];
            }
        }
#pragma unroll
        for (int s = 0; s < G::PW; ++s) {
            const int t = w + s * NW;
            if (t < G::TW) {
                const int ti = t / nTV, tj = t % nTV;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    so[D * D + (ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col()] = accW[s][r];
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < D; i += NT) so[D * D + D * DV + i] = sm.u[i];
    }
}

// ------------------------------------------------------------ summary kernel

template <typename T, int D, int DV, int C, bool DECAY, int NW>
__global__ __launch_bounds__(NW * kWave) void hla2_summary_kernel(FwdParams p) {
    using G = Hla2Cfg<T, D, DV, C, DECAY, NW>;
    constexpr int NT = G::NT, LDD = G::LDD, LDC = G::LDC;
    constexpr int nTD = G::nTD, nTV = G::nTV;
    __shared__ Hla2SumSmem<T, D, DV, C, DECAY, NW> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const int w = wave_id();
    const float g = DECAY ? p.gamma[bh % p.H] : 1.f;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;

    if (DECAY) fill_pow_table<NT>(sm.gp, G::NPOW, g);
    f32x4 accS[G::PS], accW[G::PW], accC[G::PW];
#pragma unroll
    for (int s = 0; s < G::PS; ++s) accS[s] = zero4();
#pragma unroll
    for (int s = 0; s < G::PW; ++s) { accW[s] = zero4(); accC[s] = zero4(); }
    for (int i = threadIdx.x; i < D * LDD; i += NT) sm.St[i] = from_f<T>(0.f);
    for (int i = threadIdx.x; i < D; i += NT) { sm.u[i] = 0.f; sm.m[i] = 0.f; }

    for (int c0 = t_begin; c0 < t_end; c0 += C) {
        const int cv = min(C, t_end - c0);
        __syncthreads();
        {
            constexpr int VE = Vec16<T>::N;
            for (int idx = threadIdx.x; idx < C * (D / VE); idx += NT) {
                const int r = idx / (D / VE), c = (idx % (D / VE)) * VE;
                Vec16<T> xq, xk;
                if (r < cv) {
                    xq = load16(q + (size_t)(c0 + r) * D + c);
                    xk = load16(k + (size_t)(c0 + r) * D + c);
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e) { xq.v[e] = from_f<T>(0.f); xk.v[e] = from_f<T>(0.f); }
                }
                store16(sm.Q + r * LDD + c, xq);
                store16(sm.K + r * LDD + c, xk);
                const float wr = (r < cv) ? (DECAY ? sm.gp[cv - 1 - r] : 1.f) : 0.f;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    sm.Qtw[(c + e) * LDC + r] = DECAY ? from_f<T>(to_f(xq.v[e]) * wr) : xq.v[e];
                    sm.Kt[(c + e) * LDC + r] = xk.v[e];
                    if (DECAY) sm.Ktw[(c + e) * LDC + r] = from_f<T>(to_f(xk.v[e]) * wr);
                }
            }
        }
        stage_tile<T, C, DV, NT>(v + (size_t)c0 * DV, cv, nullptr, 0, sm.Vt, LDC);
        __syncthreads();

        scores_tril<T, D, C, DECAY, NW, LDD, LDC>(sm.Q, sm.K, sm.L, sm.gp);
        f32x4 accZ[G::PZ];
#pragma unroll
        for (int s = 0; s < G::PZ; ++s) {
            const int t = w + s * NW;
            accZ[s] = zero4();
            if (t < G::TZ) {
                const int ti = t / nTD, tj = t % nTD;
                accZ[s] = mma_nt(accZ[s], sm.Q + ti * 16 * LDD, LDD, sm.St + tj * 16 * LDD, LDD, 0, D);
            }
        }
        __syncthreads();

#pragma unroll
        for (int s = 0; s < G::PZ; ++s) {
            const int t = w + s * NW;
            if (t < G::TZ) {
                const int ti = t / nTD, tj = t % nTD;
                if (DECAY) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) accZ[s][r] *= sm.gp[ti * 16 + acc_row(r) + 1];
                }
                accZ[s] = mma_nt(accZ[s], sm.L + ti * 16 * LDC, LDC, sm.Kt + tj * 16 * LDC, LDC, 0,
                                 (ti + 1) * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = ti * 16 + acc_row(r), col = tj * 16 + acc_col();
                    float wz = 0.f;
                    if (row < cv) wz = DECAY ? sm.gp[2 * (cv - 1 - row)] : 1.f;
                    sm.Ztw[col * LDC + row] = from_f<T>(accZ[s][r] * wz);
                }
            }
        }
        __syncthreads();

        const float gc = DECAY ? sm.gp[cv] : 1.f;
        const float gc2 = DECAY ? sm.gp[2 * cv] : 1.f;
        const T *KA = DECAY ? sm.Ktw : sm.Kt;
#pragma unroll
        for (int s = 0; s < G::PS; ++s) {
            const int t = w + s * NW;
            if (t < G::TS) {
                const int ti = t / nTD, tj = t % nTD;
                if (DECAY) accS[s] *= gc;
                accS[s] = mma_nt(accS[s], KA + ti * 16 * LDC, LDC, sm.Kt + tj * 16 * LDC, LDC, 0, C);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.St[(tj * 16 + acc_col()) * LDD + ti * 16 + acc_row(r)] = from_f<T>(accS[s][r]);
            }
        }
#pragma unroll
        for (int s = 0; s < G::PW; ++s) {
            const int t = w + s * NW;
            if (t < G::TW) {
                const int ti = t / nTV, tj = t % nTV;
                if (DECAY) { accW[s] *= gc2; accC[s] *= gc; }
                accW[s] = mma_nt(accW[s], sm.Ztw + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0, C);
                accC[s] = mma_nt(accC[s], sm.Qtw + ti * 16 * LDC, LDC, sm.Vt + tj * 16 * LDC, LDC, 0, C);
            }
        }
        for (int i = threadIdx.x; i < D; i += NT) {
            float su = 0.f, sq = 0.f;
            for (int c = 0; c < C; ++c) {
                su += to_f(sm.Ztw[i * LDC + c]);
                sq += to_f(sm.Qtw[i * LDC + c]);
            }
            sm.u[i] = gc2 * sm.u[i] + su;
            sm.m[i] = gc * sm.m[i] + sq;
        }
    }
    __syncthreads();

    // summary [X = S | Y = C | N = W | y = m | nv = u]
    float *e = p.ws + ws_elem(bh, 0, p.spad, seg, G::SUMF);
#pragma unroll
    for (int s = 0; s < G::PS; ++s) {
        const int t = w + s * NW;
        if (t < G::TS) {
            const int ti = t / nTD, tj = t % nTD;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                e[(ti * 16 + acc_row(r)) * D + tj * 16 + acc_col()] = accS[s][r];
        }
    }
#pragma unroll
    for (int s = 0; s < G::PW; ++s) {
        const int t = w + s * NW;
        if (t < G::TW) {
            const int ti = t / nTV, tj = t % nTV;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = (ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col();
                e[D * D + idx] = accC[s][r];
                e[D * D + D * DV + idx] = accW[s][r];
            }
        }
    }
    for (int i = threadIdx.x; i < D; i += NT) {
        e[D * D + 2 * D * DV + i] = sm.m[i];
        e[D * D + 2 * D * DV + D + i] = sm.u[i];
    }
}

}  // namespace hla
