// step_kernel.h -- one streaming (decode) step of HLA-2 / AHLA per (b,h).
//
// Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
// gist.science/es/paper/2510.27258, sections "1. HLA de Segundo Orden" and
// "Resultados y Afirmaciones": a constant-size state per head and an
// O(d^2 + d dv) update per token, independent of the sequence length;
// section "2. ... (AHLA)" for the asymmetric summaries.
//
// HLA-2: S <- g S + k k^T ; z = S q ; W <- g^2 W + z v^T ; u <- g^2 u + z ;
//        o = q^T W  (ratio: / q^T u)
// AHLA : P <- g P + k v^T ; y = P^T q ; E <- g E + k y^T ; mK <- g mK + k ;
//        nk <- g nk + k (q . mK) ; o = q^T E  (ratio: / q^T nk)
//        (every summary decays by g per token; g = 1 without a decay)
// HLA3 : P <- g P + k v^T ; y = P^T q ; S <- g S + k k^T ; z = S q ;
//        W <- g^3 W + z y^T ; o = q^T W  (hla3_step_kernel; section "3. HLA de
//        Tercer Orden": the third-order operator read as tril(L L^T) L V, every
//        moment decayed by g per token; the ratio form runs the same step on
//        unit values (1, 0, ..., 0) in its second state block and divides)
//
// One workgroup of NT threads per (b,h).  The state is read once and written
// once (fp32, row-major), with consecutive threads on consecutive columns so
// every access is coalesced.  Every thread issues all of its state loads at
// the start, so the step costs one memory round trip plus its reductions.
#pragma once

#include "device_common.h"
#include "params.h"

namespace hla {

template <typename T, int D, int DV, int MODE, int NT>
__global__ __launch_bounds__(NT) void step_kernel(StepParams p) {
    constexpr bool AHLA = MODE == kStepAhla;
    static_assert(MODE != kStepHla3, "third order: hla3_step_kernel");
    constexpr int RG = NT / DV;     // row groups of the column-parallel passes
    constexpr int RPT = D / RG;     // rows per thread in those passes
    constexpr int TPR = NT / D;     // threads per row of the S pass (HLA-2)
    constexpr int CPT = D / TPR;    // S columns per thread
    static_assert(NT % DV == 0 && NT % D == 0 && D % RG == 0 && D % TPR == 0, "block shape");
    __shared__ float sq[D], sk[D], sv[DV], sz[D], sy[DV];
    __shared__ float part[RG][DV];
    __shared__ float red[NT / kWave];

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float g = p.gamma[gamma_slot(bh, p.H)];
    const float g2 = g * g;
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * DV;
    constexpr int STF = AHLA ? ahla_state_floats(D, DV) : hla2_state_floats(D, DV);
    float *st = p.state + (size_t)bh * STF;
    const int col = tid % DV, rg = tid / DV;

    auto block_sum = [&](float x) -> float {
        for (int m = kWave / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m);
        if ((tid & (kWave - 1)) == 0) red[tid / kWave] = x;
        __syncthreads();
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NT / kWave; ++i) s += red[i];
        __syncthreads();
        return s;
    };

    if (!AHLA) {
        float *S = st, *W = st + D * D, *u = st + D * D + D * DV;
        const int row = tid / TPR, sub = tid % TPR;
        float sv_[CPT], wv[RPT], uv = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) sv_[i] = S[row * D + sub + i * TPR];
#pragma unroll
        for (int i = 0; i < RPT; ++i) wv[i] = W[(rg + i * RG) * DV + col];
        if (tid < D) uv = u[tid];
        for (int i = tid; i < D; i += NT) { sq[i] = to_f(q[i]); sk[i] = to_f(k[i]); }
        for (int j = tid; j < DV; j += NT) sv[j] = to_f(v[j]);
        __syncthreads();
        // S <- g S + k k^T ; z = S q
        float zp = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = sub + i * TPR;
            const float sn = g * sv_[i] + sk[row] * sk[c];
            S[row * D + c] = sn;
            zp += sn * sq[c];
        }
        for (int m = TPR / 2; m >= 1; m >>= 1) zp += __shfl_xor(zp, m, TPR);
        if (sub == 0) sz[row] = zp;
        __syncthreads();
        // W <- g^2 W + z v^T ; partial o = q^T W
        float op = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + i * RG;
            const float wn = g2 * wv[i] + sz[r] * sv[col];
            W[r * DV + col] = wn;
            op += sq[r] * wn;
        }
        part[rg][col] = op;
        // u <- g^2 u + z ; den = q^T u
        float dp = 0.f;
        if (tid < D) {
            const float un = g2 * uv + sz[tid];
            u[tid] = un;
            dp = sq[tid] * un;
        }
        const float den = block_sum(dp);   // its barrier also publishes part[]
        if (tid < DV) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < RG; ++i) s += part[i][tid];
            if (p.ratio) s = s / den;
            o[tid] = from_f<T>(s);
        }
    } else {
        float *P = st, *E = st + D * DV, *mK = st + 2 * D * DV, *nk = mK + D;
        float pv[RPT], ev[RPT], mkv = 0.f, nkv = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            pv[i] = P[(rg + i * RG) * DV + col];
            ev[i] = E[(rg + i * RG) * DV + col];
        }
        if (tid < D) {
            mkv = mK[tid];
            nkv = nk[tid];
        }
        for (int i = tid; i < D; i += NT) { sq[i] = to_f(q[i]); sk[i] = to_f(k[i]); }
        for (int j = tid; j < DV; j += NT) sv[j] = to_f(v[j]);
        __syncthreads();
        // P <- g P + k v^T ; partial y = P^T q
        float yp = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + i * RG;
            const float pn = g * pv[i] + sk[r] * sv[col];
            P[r * DV + col] = pn;
            yp += sq[r] * pn;
        }
        part[rg][col] = yp;
        // mK <- g mK + k ; s = q . mK
        float sp = 0.f;
        if (tid < D) {
            mkv = g * mkv + sk[tid];
            mK[tid] = mkv;
            sp = sq[tid] * mkv;
        }
        const float s_all = block_sum(sp);   // its barrier also publishes part[]
        if (tid < DV) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < RG; ++i) s += part[i][tid];
            sy[tid] = s;
        }
        __syncthreads();
        // E <- g E + k y^T ; partial o = q^T E
        float op = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + i * RG;
            const float en = g * ev[i] + sk[r] * sy[col];
            E[r * DV + col] = en;
            op += sq[r] * en;
        }
        part[rg][col] = op;
        // nk <- g nk + k s ; den = q . nk
        float dp = 0.f;
        if (tid < D) {
            nkv = g * nkv + sk[tid] * s_all;
            nk[tid] = nkv;
            dp = sq[tid] * nkv;
        }
        const float den = block_sum(dp);
        if (tid < DV) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < RG; ++i) s += part[i][tid];
            if (p.ratio) s = s / den;
            o[tid] = from_f<T>(s);
        }
    }
}

}  // namespace hla

namespace hla {

// The unnormalised AHLA step split over column slices of 16 value columns:
// workgroup (bh, slice) owns columns [16 slice, 16 slice + 16) of P and E.
// With the old state, every quantity the step needs is one dot product with
// q (or k):
//     y_j = (g P + k v^T)[:, j] . q = g (P[:, j] . q) + (k . q) v_j
//     o_j = (g E + k y^T)[:, j] . q = g (E[:, j] . q) + (k . q) y_j
// so the workgroup forms the column sums P.q, E.q, k.q (and q.mK for the
// slice that owns mK, nk) in one reduction -- one barrier -- and writes
// P' = g P + k v^T (which needs no sum) before it, E' = g E + k y^T after.
// mK <- g mK + k, nk <- g nk + k (q . mK') belong to slice 0 alone, so no
// two workgroups touch the same state word.  (The ratio form needs q . nk in
// every slice and keeps the one-workgroup kernel above.)  At d = 64 that is
// four workgroups per head, so a decode step of few heads reaches more of
// the chip, and every state load is issued at the kernel's start.
template <typename T, int D, int DV, int NT, int SW = 16>   // SW: columns per slice
__global__ __launch_bounds__(NT) void ahla_step_sliced_kernel(StepParams p) {
    constexpr int RG = NT / SW;         // row groups
    constexpr int RPT = D / RG;         // rows per thread
    constexpr int NWV = NT / kWave;     // waves
    constexpr int RGW = kWave / SW;     // row groups per wave
    static_assert(DV % SW == 0 && NT % SW == 0 && D % RG == 0 && kWave % SW == 0, "block shape");
    __shared__ float red[NWV][4][SW];

    const int nsl = DV / SW;
    const int bh = blockIdx.x / nsl, slice = blockIdx.x % nsl;
    const int tid = threadIdx.x;
    const int col = tid % SW, rg = tid / SW;
    const int j = slice * SW + col;     // this thread's value column
    const float g = p.gamma[gamma_slot(bh, p.H)];
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * DV;
    float *st = p.state + (size_t)bh * ahla_state_floats(D, DV);
    float *P = st, *E = st + D * DV, *mK = st + 2 * D * DV, *nk = mK + D;

    // every load first: this thread's rows r = rg + i RG of column j
    float pv[RPT], ev[RPT], qv[RPT], kv[RPT], mv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        pv[i] = P[r * DV + j];
        ev[i] = E[r * DV + j];
        qv[i] = to_f(q[r]);
        kv[i] = to_f(k[r]);
        mv[i] = slice == 0 ? mK[r] : 0.f;   // only slice 0 reads or writes mK
    }
    const float vj = to_f(v[j]);

    // P' = g P + k v^T needs no sum
    float sums[4] = {0.f, 0.f, 0.f, 0.f};   // P.q, E.q, k.q, q.mK over this thread's rows
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        P[r * DV + j] = g * pv[i] + kv[i] * vj;
        sums[0] += qv[i] * pv[i];
        sums[1] += qv[i] * ev[i];
        sums[2] += qv[i] * kv[i];
        sums[3] += qv[i] * mv[i];
    }
    // over the row groups of this wave (lanes 16 apart share the column),
    // then over the waves through LDS
#pragma unroll
    for (int x = 0; x < 4; ++x) {
#pragma unroll
        for (int m = SW; m < kWave; m <<= 1) sums[x] += __shfl_xor(sums[x], m);
    }
    const int wv = tid / kWave;
    if ((tid % kWave) < SW) {
#pragma unroll
        for (int x = 0; x < 4; ++x) red[wv][x][col] = sums[x];
    }
    __syncthreads();
    float tot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWV; ++w)
#pragma unroll
        for (int x = 0; x < 4; ++x) tot[x] += red[w][x][col];
    const float kq = tot[2];
    const float yj = g * tot[0] + kq * vj;
    // E' = g E + k y^T ; o_j
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        E[r * DV + j] = g * ev[i] + kv[i] * yj;
    }
    if (rg == 0) o[j] = from_f<T>(g * tot[1] + kq * yj);
    if (slice == 0 && col == 0) {
        // mK' = g mK + k ; nk' = g nk + k (q . mK'), q . mK' = g (q . mK) + k . q
        const float qm = g * tot[3] + kq;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + i * RG;
            mK[r] = g * mv[i] + kv[i];
            nk[r] = g * nk[r] + kv[i] * qm;
        }
    }
}

}  // namespace hla

namespace hla {

// Third-order step, one workgroup per (b,h): for each chain (the values v;
// for the ratio form also the unit values (1, 0, ..., 0), whose state block
// follows the first one)
//   P <- g P + k v^T ; y = P^T q ; S <- g S + k k^T ; z = S q ;
//   W <- g^3 W + z y^T ; o = q^T W
// and the ratio form divides the first chain's o by the second's o[0].  The
// u part of each second-order block is not used by third order.
template <typename T, int D, int DV, int NT>
__global__ __launch_bounds__(NT) void hla3_step_kernel(StepParams p) {
    constexpr int RG = NT / DV;     // row groups of the column-parallel passes
    constexpr int RPT = D / RG;     // rows per thread in those passes
    constexpr int TPR = NT / D;     // threads per row of the S pass
    constexpr int CPT = D / TPR;    // S columns per thread
    static_assert(NT % DV == 0 && NT % D == 0 && D % RG == 0 && D % TPR == 0, "block shape");
    __shared__ float sq[D], sk[D], sv[DV], sz[D], sy[DV];
    __shared__ float part[RG][DV];
    __shared__ float sden;

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float g = p.gamma[gamma_slot(bh, p.H)];
    const float g3 = g * g * g;
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * DV;
    const size_t chain_floats = (size_t)p.BH * hla3_state_floats(D, DV);
    const int col = tid % DV, rg = tid / DV;
    const int row = tid / TPR, sub = tid % TPR;

    for (int i = tid; i < D; i += NT) { sq[i] = to_f(q[i]); sk[i] = to_f(k[i]); }
    float onum = 0.f;
    const int nchain = p.ratio ? 2 : 1;
    for (int chain = 0; chain < nchain; ++chain) {
        float *P = p.state + chain * chain_floats + (size_t)bh * D * DV;
        float *S = p.state + chain * chain_floats + (size_t)p.BH * D * DV +
                   (size_t)bh * hla2_state_floats(D, DV);
        float *W = S + D * D;
        float pv[RPT], wv[RPT], svv[CPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            pv[i] = P[(rg + i * RG) * DV + col];
            wv[i] = W[(rg + i * RG) * DV + col];
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) svv[i] = S[row * D + sub + i * TPR];
        for (int j = tid; j < DV; j += NT) sv[j] = chain == 0 ? to_f(v[j]) : (j == 0 ? 1.f : 0.f);
        __syncthreads();
        // P <- g P + k v^T ; partial y = P^T q
        float yp = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + i * RG;
            const float pn = g * pv[i] + sk[r] * sv[col];
            P[r * DV + col] = pn;
            yp += sq[r] * pn;
        }
        part[rg][col] = yp;
        // S <- g S + k k^T ; z = S q
        float zp = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = sub + i * TPR;
            const float sn = g * svv[i] + sk[row] * sk[c];
            S[row * D + c] = sn;
            zp += sn * sq[c];
        }
        for (int m = TPR / 2; m >= 1; m >>= 1) zp += __shfl_xor(zp, m, TPR);
        if (sub == 0) sz[row] = zp;
        __syncthreads();
        if (tid < DV) {
            float y = 0.f;
#pragma unroll
            for (int i = 0; i < RG; ++i) y += part[i][tid];
            sy[tid] = y;
        }
        __syncthreads();
        // W <- g^3 W + z y^T ; partial o = q^T W
        float op = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + i * RG;
            const float wn = g3 * wv[i] + sz[r] * sy[col];
            W[r * DV + col] = wn;
            op += sq[r] * wn;
        }
        part[rg][col] = op;
        __syncthreads();
        if (tid < DV) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < RG; ++i) s += part[i][tid];
            if (chain == 0) onum = s;
            else if (tid == 0) sden = s;
        }
        __syncthreads();   // part, sv reused by the next chain; sden published
    }
    if (tid < DV) o[tid] = from_f<T>(p.ratio ? onum / sden : onum);
}

}  // namespace hla
