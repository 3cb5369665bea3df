// scan_kernel.h -- exclusive Blelloch scan of segment summaries under the
// semidirect-product combine (gfx950).
//
// Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
// gist.science/es/paper/2510.27258, section "4. Entrenamiento Paralelo
// mediante Escaneos Asociativos": segments are concatenated by an associative
// semidirect-product operator whose cross terms pair one segment's key moment
// with the other's query-value moment, and an exclusive Blelloch scan over the
// segment summaries reproduces the serial recurrence exactly.
//
// Summary = (X, Y, N, y, nv) (layout in params.h).  Combine, A earlier than B,
// a = g^(length of B) (1 for AHLA):
//   HLA-2: X = a X_A + X_B, Y = a Y_A + Y_B, y = a y_A + y_B,
//          N = a^2 N_A + N_B + a X_A Y_B,  nv = a^2 nv_A + nv_B + a X_A y_B
//   AHLA : X = X_A + X_B, Y = Y_A + Y_B, y = y_A + y_B,
//          N = N_A + N_B + X_B Y_A,        nv = nv_A + nv_B + X_B y_A
// The identity is the zero summary.
//
// One workgroup per (b,h).  The up-sweep combines in place in the "e" array;
// the down-sweep writes the exclusive prefixes into the separate "p" array
// (p[left] <- p[right]; p[right] <- p[right] (+) e[left]).  The up-sweep
// skips every combine that only feeds the total (the pairs ending at the last
// slot), since an exclusive scan discards it.  Finally the caller's initial
// state, if any, is folded in front of every prefix.  All pairs of one tree
// level run concurrently across the waves.
#pragma once

#include "device_common.h"
#include "params.h"

namespace hla {

// acc = Xc[ti*16 .. +16][0:K] * Yc[0:K][tj*16 .. +16], fp32 operands read from
// global memory.  F32: exact fp32 MFMA.  Otherwise each operand is split into
// bf16 hi + lo parts and the product is hi*hi + hi*lo + lo*hi (relative error
// about 2^-16 per product, far below the bf16 path's own rounding).
template <bool F32, int K>
__device__ __forceinline__ f32x4 cross_tile(const float *Xc, int ldx, const float *Yc, int ldy,
                                            int ti, int tj) {
    const int l = lane_id();
    const int r = l & 15, gq = l >> 4;
    f32x4 acc = zero4();
    if constexpr (F32) {
        const float *a = Xc + (ti * 16 + r) * ldx + gq;
        const float *b = Yc + gq * ldy + tj * 16 + r;
#pragma unroll 4
        for (int k = 0; k < K; k += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k], b[k * ldy], acc, 0, 0, 0);
    } else {
        const float *a = Xc + (ti * 16 + r) * ldx;
        const float *b = Yc + tj * 16 + r;
        int k = 0;
#pragma unroll
        for (; k + 32 <= K; k += 32) {
            bf16x8 ah, al, bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = a[k + gq * 8 + e];
                const bf16 xh = (bf16)x;
                ah[e] = xh;
                al[e] = (bf16)(x - (float)xh);
                const float y = b[(k + gq * 8 + e) * ldy];
                const bf16 yh = (bf16)y;
                bh[e] = yh;
                bl[e] = (bf16)(y - (float)yh);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        }
        if constexpr (K % 32 == 16) {
            union { bf16 h[4]; i16x4 v; } ah, al, bh, bl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = a[k + gq * 4 + e];
                const bf16 xh = (bf16)x;
                ah.h[e] = xh;
                al.h[e] = (bf16)(x - (float)xh);
                const float y = b[(k + gq * 4 + e) * ldy];
                const bf16 yh = (bf16)y;
                bh.h[e] = yh;
                bl.h[e] = (bf16)(y - (float)yh);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah.v, bh.v, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah.v, bl.v, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al.v, bh.v, acc, 0, 0, 0);
        }
    }
    return acc;
}

template <int D, int DV>
struct SumOfs {
    static constexpr int X = 0, Y = D * D, N = D * D + D * DV, y = D * D + 2 * D * DV,
                         nv = D * D + 2 * D * DV + D;
};

// dst.N = a2 * A.N + B.N + a * Xc Yc ;  dst.nv = a2 * A.nv + B.nv + a * Xc yc
// for `npair` pairs given by pair(j, &A, &B, &dst, &a).  Xc, Yc, yc come from
// B / A as the variant says.  Waves take (pair, 16-row slab) items; threads
// take (pair, row) items of nv.  dst may equal B (each element is read and
// written by one owner) but A and B are not written.
template <bool F32, int D, int DV, bool HLA2, int NW, typename PairFn>
__device__ __forceinline__ void cross_phase(int npair, PairFn pair) {
    using O = SumOfs<D, DV>;
    constexpr int NT = NW * kWave, nTD = D / 16, nTV = DV / 16;
    const int w = wave_id();
    for (int it = w; it < npair * nTD; it += NW) {
        const int j = it / nTD, ti = it % nTD;
        const float *A, *B;
        float *Dst;
        float a;
        pair(j, A, B, Dst, a);
        const float *Xc = HLA2 ? A + O::X : B + O::X;
        const float *Yc = HLA2 ? B + O::Y : A + O::Y;
        const float a2 = a * a;
        for (int tj = 0; tj < nTV; ++tj) {
            const f32x4 c = cross_tile<F32, D>(Xc, D, Yc, DV, ti, tj);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = (ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col();
                Dst[O::N + idx] = a2 * A[O::N + idx] + B[O::N + idx] + a * c[r];
            }
        }
    }
    for (int it = threadIdx.x; it < npair * D; it += NT) {
        const int j = it / D, row = it % D;
        const float *A, *B;
        float *Dst;
        float a;
        pair(j, A, B, Dst, a);
        const float *Xc = HLA2 ? A + O::X : B + O::X;
        const float *yc = HLA2 ? B + O::y : A + O::y;
        float s = 0.f;
        for (int c = 0; c < D; ++c) s += Xc[row * D + c] * yc[c];
        Dst[O::nv + row] = a * a * A[O::nv + row] + B[O::nv + row] + a * s;
    }
}

// dst.{X,Y,y} = a * A.{X,Y,y} + B.{X,Y,y}
template <int D, int DV, int NW, typename PairFn>
__device__ __forceinline__ void linear_phase(int npair, PairFn pair) {
    using O = SumOfs<D, DV>;
    constexpr int NT = NW * kWave;
    constexpr int NX = D * D + D * DV;   // X and Y are contiguous
    constexpr int PER = NX + D;
    for (int it = threadIdx.x; it < npair * PER; it += NT) {
        const int j = it / PER, x = it % PER;
        const float *A, *B;
        float *Dst;
        float a;
        pair(j, A, B, Dst, a);
        const int idx = x < NX ? x : O::y + (x - NX);
        Dst[idx] = a * A[idx] + B[idx];
    }
}

template <bool F32, int D, int DV, bool HLA2, int NW>
__global__ __launch_bounds__(NW * kWave) void scan_kernel(FwdParams p) {
    using O = SumOfs<D, DV>;
    constexpr int NT = NW * kWave;
    constexpr int SUMF = summary_floats(D, DV);
    const int bh = blockIdx.x;
    const int spad = p.spad, nreal = p.nseg - 1;  // e[0 .. nreal-1] hold real summaries
    const float g = HLA2 ? p.gamma[bh % p.H] : 1.f;
    float *E = p.ws + ws_elem(bh, 0, spad, 0, SUMF);
    float *Pr = p.ws + ws_elem(bh, 1, spad, 0, SUMF);
    // tokens covered by segments [lo, hi] of e (slots >= nreal are identities)
    auto span = [&](int lo, int hi) -> long {
        hi = min(hi, nreal - 1);
        return hi >= lo ? (long)(hi - lo + 1) * p.seg_len : 0L;
    };

    for (size_t idx = threadIdx.x; idx < (size_t)(spad - nreal) * SUMF; idx += NT)
        E[(size_t)nreal * SUMF + idx] = 0.f;
    for (size_t idx = threadIdx.x; idx < SUMF; idx += NT) Pr[(size_t)(spad - 1) * SUMF + idx] = 0.f;
    __syncthreads();

    // ---- up-sweep: e[i] <- e[i-s] (+) e[i], i = 2s-1, 4s-1, ..., < spad-1
    for (int s = 1; s < spad; s <<= 1) {
        const int npair = spad / (2 * s) - 1;
        if (npair <= 0) continue;
        auto pair = [&](int j, const float *&A, const float *&B, float *&Dst, float &a) {
            const int i = (j + 1) * 2 * s - 1;
            A = E + (size_t)(i - s) * SUMF;
            B = E + (size_t)i * SUMF;
            Dst = E + (size_t)i * SUMF;
            a = HLA2 ? pow_int(g, span(i - s + 1, i)) : 1.f;
        };
        cross_phase<F32, D, DV, HLA2, NW>(npair, pair);
        __syncthreads();
        linear_phase<D, DV, NW>(npair, pair);
        __syncthreads();
    }

    // ---- down-sweep: p[i-s] <- p[i];  p[i] <- p[i] (+) e[i-s]
    for (int s = spad >> 1; s >= 1; s >>= 1) {
        const int npair = spad / (2 * s);
        for (size_t it = threadIdx.x; it < (size_t)npair * SUMF; it += NT) {
            const int j = (int)(it / SUMF), x = (int)(it % SUMF);
            const int i = (j + 1) * 2 * s - 1;
            Pr[(size_t)(i - s) * SUMF + x] = Pr[(size_t)i * SUMF + x];
        }
        __syncthreads();
        auto pair = [&](int j, const float *&A, const float *&B, float *&Dst, float &a) {
            const int i = (j + 1) * 2 * s - 1;
            A = Pr + (size_t)(i - s) * SUMF;   // copy of the old p[i]
            B = E + (size_t)(i - s) * SUMF;    // aggregate of the left subtree
            Dst = Pr + (size_t)i * SUMF;
            a = HLA2 ? pow_int(g, span(i - 2 * s + 1, i - s)) : 1.f;
        };
        cross_phase<F32, D, DV, HLA2, NW>(npair, pair);
        linear_phase<D, DV, NW>(npair, pair);
        __syncthreads();
    }

    // ---- fold the caller's initial state in front of every prefix
    if (p.state_in) {
        const int STF = HLA2 ? hla2_state_floats(D, DV) : ahla_state_floats(D, DV);
        const float *st = p.state_in + (size_t)bh * STF;
        const int nseg = p.nseg;
        const int w = wave_id();
        constexpr int nTD = D / 16, nTV = DV / 16;
        if (HLA2) {
            // state_in = (S, W, u) with C = m = 0:  X += a S, N = a^2 W + N + a S Y,
            // nv = a^2 u + nv + a S y ;  Y, y unchanged
            const float *S = st, *W = st + D * D, *u = st + D * D + D * DV;
            for (int it = w; it < nseg * nTD; it += NW) {
                const int s = it / nTD, ti = it % nTD;
                float *Bp = Pr + (size_t)s * SUMF;
                const float a = pow_int(g, (long)s * p.seg_len);
                for (int tj = 0; tj < nTV; ++tj) {
                    const f32x4 c = cross_tile<F32, D>(S, D, Bp + O::Y, DV, ti, tj);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int idx = (ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col();
                        Bp[O::N + idx] = a * a * W[idx] + Bp[O::N + idx] + a * c[r];
                    }
                }
            }
            for (int it = threadIdx.x; it < nseg * D; it += NT) {
                const int s = it / D, row = it % D;
                float *Bp = Pr + (size_t)s * SUMF;
                const float a = pow_int(g, (long)s * p.seg_len);
                float acc = 0.f;
                for (int c = 0; c < D; ++c) acc += S[row * D + c] * Bp[O::y + c];
                Bp[O::nv + row] = a * a * u[row] + Bp[O::nv + row] + a * acc;
            }
            for (int it = threadIdx.x; it < nseg * D * D; it += NT) {
                const int s = it / (D * D), x = it % (D * D);
                float *Bp = Pr + (size_t)s * SUMF;
                Bp[O::X + x] = pow_int(g, (long)s * p.seg_len) * S[x] + Bp[O::X + x];
            }
        } else {
            // state_in = (P, E, mK, nk):  Y += P, y += mK, N = E + N + M P,
            // nv = nk + nv + M mK  (M = X of the prefix)
            const float *P = st, *Ein = st + D * DV, *mK = st + 2 * D * DV, *nk = mK + D;
            for (int it = w; it < nseg * nTD; it += NW) {
                const int s = it / nTD, ti = it % nTD;
                float *Bp = Pr + (size_t)s * SUMF;
                for (int tj = 0; tj < nTV; ++tj) {
                    const f32x4 c = cross_tile<F32, D>(Bp + O::X, D, P, DV, ti, tj);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int idx = (ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col();
                        Bp[O::N + idx] = Ein[idx] + Bp[O::N + idx] + c[r];
                    }
                }
            }
            for (int it = threadIdx.x; it < nseg * D; it += NT) {
                const int s = it / D, row = it % D;
                float *Bp = Pr + (size_t)s * SUMF;
                float acc = 0.f;
                for (int c = 0; c < D; ++c) acc += Bp[O::X + row * D + c] * mK[c];
                Bp[O::nv + row] = nk[row] + Bp[O::nv + row] + acc;
            }
            __syncthreads();  // the M reads above precede nothing that writes M; Y, y next
            for (int it = threadIdx.x; it < nseg * (D * DV + D); it += NT) {
                const int s = it / (D * DV + D), x = it % (D * DV + D);
                float *Bp = Pr + (size_t)s * SUMF;
                if (x < D * DV) Bp[O::Y + x] += P[x];
                else Bp[O::y + (x - D * DV)] += mK[x - D * DV];
            }
        }
    }
}

}  // namespace hla
