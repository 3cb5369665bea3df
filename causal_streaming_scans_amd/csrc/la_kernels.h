// la_kernels.h -- chunked first-order causal linear attention on gfx950, the
// building block of the HLA-2 backward pass.
//
//   out_t = add_t + sum_{s <= t} g^(t-s) (a_t . b_s) c_s           (forward time)
//
// and the same over the reversed sequence (s >= t, weight g^(s-t)) when
// `reverse` is set: logical token l is physical row n-1-l, so an anti-causal
// pass is the causal pass run backwards through memory.
//
// The gradient of HLA-2 is a chain of such passes.  With z_t = S^K_t q_t =
// sum_{i<=t} g^(t-i) (q_t . k_i) k_i (the key read-out of page section "1. HLA
// de Segundo Orden"), the masked operator is two chained linear attentions,
// Z = LA_g(Q, K, K) and O = LA_{g^2}(Q, Z, V), and the chain rule through each
// one gives three more of the same form (see hla_api.cpp).
//
// Parallel form (page section "4. Entrenamiento Paralelo mediante Escaneos
// Asociativos", first order): the state S = sum_s g^(.) b_s c_s^T is additive,
// so the sequence is cut into segments; a summary launch forms each segment's
// S from zero, and each main workgroup folds the summaries of the segments
// before its own (S <- g^len S + S_seg) and then runs its chunks.
//
// Per chunk of C tokens (one workgroup, NW = 4 waves):
//   P     = D_g * tril(A_c B_c^T)                           (C x C, in LDS)
//   out^T = C_c^T P^T + S^T A_c^T diag(g^(tau+1)) [+ add]   (written from registers)
//   S     = g^C S + (B_c^T diag(g^(C-1-sigma))) C_c         (fp32, in registers)
// Products use the "NT" MFMA form of device_common.h with both operands
// row-major along k in LDS: c and the weighted b are staged transposed
// ([feature][token]) next to the row-major a and b.
#pragma once

#include "device_common.h"
#include "params.h"

namespace hla {

template <typename T, int D, int C>
struct LaLds {
    using TR = PadTile<T, D>;    // [C][D] a, b rows; [D][D] state copy St[j][i] = S[i][j]
    using TT = PadTile<T, C>;    // [D][C] transposed c and weighted b; [C][C] scores
    T a[C * TR::LD];
    T b[C * TR::LD];
    T ct[D * TT::LD];
    T btw[D * TT::LD];
    T p[C * TT::LD];
    T st[D * TR::LD];
    float pw[C + 1];             // g^e, e = 0..C
};

template <typename T, int D, int C>
struct LaCfg {
    static constexpr int NW = 4, NT = NW * kWave;
    static constexpr int TR = C / 16;          // token tiles per chunk
    static constexpr int TD = D / 16;          // feature tiles
    static constexpr int NS = TD * TD;         // state tiles
    static constexpr int SPW = (NS + NW - 1) / NW;   // state tiles per wave
    static constexpr int blocks() {
        constexpr size_t lds = sizeof(LaLds<T, D, C>);
        return lds <= 40 * 1024 ? 3 : (lds <= 80 * 1024 ? 2 : 1);
    }
};

// Stage the chunk whose first logical token is l0: a, b row-major, c and
// g^(C-1-sigma) b transposed.  Rows past the end of the sequence are zeros.
template <typename T, int D, int C>
__device__ __forceinline__ void la_stage(const LaParams &p, size_t head_row, int l0,
                                         LaLds<T, D, C> &s) {
    using L = LaLds<T, D, C>;
    constexpr int VE = Vec16<T>::N, VPR = D / VE, NV = C * VPR;
    constexpr int NT = LaCfg<T, D, C>::NT;
    const T *A = static_cast<const T *>(p.a);
    const T *B = static_cast<const T *>(p.b);
    const T *Cv = static_cast<const T *>(p.c);
    for (int idx = threadIdx.x; idx < NV; idx += NT) {
        const int r = idx / VPR, col = (idx % VPR) * VE;
        const int l = l0 + r;
        Vec16<T> xa, xb, xc;
        if (l < p.n) {
            const size_t row = head_row + (size_t)(p.reverse ? p.n - 1 - l : l);
            xa = load16(A + row * D + col);
            xb = load16(B + row * D + col);
            xc = load16(Cv + row * D + col);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) xa.v[e] = xb.v[e] = xc.v[e] = from_f<T>(0.f);
        }
        store16(s.a + L::TR::off(r, col), xa);
        store16(s.b + L::TR::off(r, col), xb);
        const float w = s.pw[C - 1 - r];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            s.ct[L::TT::off(col + e, r)] = xc.v[e];
            s.btw[L::TT::off(col + e, r)] = from_f<T>(to_f(xb.v[e]) * w);
        }
    }
}

// The state tiles of this wave: tile m = wave + NW*i covers S rows
// 16*(m / TD) .., columns 16*(m % TD) ..
template <typename T, int D, int C>
struct LaState {
    using Cfg = LaCfg<T, D, C>;
    f32x4 acc[Cfg::SPW];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < Cfg::SPW; ++i) acc[i] = zero4();
    }
    // S <- g^C S + Btw Ct^T (products of the staged chunk)
    __device__ __forceinline__ void advance(const LaLds<T, D, C> &s, float gC, int w) {
        using L = LaLds<T, D, C>;
#pragma unroll
        for (int i = 0; i < Cfg::SPW; ++i) {
            const int m = w + Cfg::NW * i;
            if (m < Cfg::NS) {
                const int si = m / Cfg::TD, sj = m % Cfg::TD;
                RowFrags<T, C> fc;
                fc.template load_t<typename L::TT>(s.ct + L::TT::off(16 * sj, 0));
                f32x4 a = acc[i];
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] *= gC;
                acc[i] = mma_nt_ft<typename L::TT, C>(a, s.btw + L::TT::off(16 * si, 0), fc);
            }
        }
    }
    // St[j][i] = S[i][j], rounded to T
    __device__ __forceinline__ void store_copy(LaLds<T, D, C> &s, int w) const {
        using L = LaLds<T, D, C>;
        const int l = lane_id(), g = l >> 4;
#pragma unroll
        for (int i = 0; i < Cfg::SPW; ++i) {
            const int m = w + Cfg::NW * i;
            if (m < Cfg::NS) {
                const int si = m / Cfg::TD, sj = m % Cfg::TD;
                store4(s.st + L::TR::off(16 * sj + (l & 15), 16 * si + 4 * g), acc[i]);
            }
        }
    }
};

// Summary of segment seg (< nseg-1): its state from zero, decayed to its end,
// into p.sums.  Grid: (nseg-1) * BH workgroups, heads fastest.
template <typename T, int D, int C>
__global__ __launch_bounds__((LaCfg<T, D, C>::NT), (LaCfg<T, D, C>::blocks()))
void la_summary_kernel(LaParams p) {
    using Cfg = LaCfg<T, D, C>;
    __shared__ LaLds<T, D, C> s;
    const int L = blockIdx.x;
    const int bh = L % p.BH, seg = L / p.BH;
    const int w = wave_id();
    const float g = p.gamma[gamma_slot(bh, p.H)];
    fill_pow_table<Cfg::NT>(s.pw, C + 1, g);
    __syncthreads();
    const float gC = s.pw[C];
    const size_t head_row = (size_t)bh * p.n;
    const int l_begin = seg * p.seg_len;
    const int l_end = min(p.n, l_begin + p.seg_len);
    LaState<T, D, C> S;
    S.zero();
    for (int l0 = l_begin; l0 < l_end; l0 += C) {
        la_stage<T, D, C>(p, head_row, l0, s);
        __syncthreads();
        S.advance(s, gC, w);
        __syncthreads();
    }
    float *dst = p.sums + ((size_t)bh * (p.nseg - 1) + seg) * (D * D);
    const int l = lane_id(), gq = l >> 4;
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
        const int m = w + Cfg::NW * i;
        if (m < Cfg::NS) {
            const int si = m / Cfg::TD, sj = m % Cfg::TD;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * si + 4 * gq + r) * D + 16 * sj + (l & 15)] = S.acc[i][r];
        }
    }
}

// Main pass over segment seg.  Grid: nseg * BH workgroups, heads fastest.
template <typename T, int D, int C>
__global__ __launch_bounds__((LaCfg<T, D, C>::NT), (LaCfg<T, D, C>::blocks()))
void la_forward_kernel(LaParams p) {
    using Cfg = LaCfg<T, D, C>;
    using Ls = LaLds<T, D, C>;
    __shared__ Ls s;
    const int L = blockIdx.x;
    const int bh = L % p.BH, seg = L / p.BH;
    const int w = wave_id();
    const int l = lane_id(), gq = l >> 4, cl = l & 15;
    const float g = p.gamma[gamma_slot(bh, p.H)];
    fill_pow_table<Cfg::NT>(s.pw, C + 1, g);
    const size_t head_row = (size_t)bh * p.n;
    const int l_begin = seg * p.seg_len;
    const int l_end = min(p.n, l_begin + p.seg_len);

    // carried state: the summaries of the segments before this one, in order
    LaState<T, D, C> S;
    S.zero();
    if (seg > 0) {
        const float gL = pow_int(g, p.seg_len);
        for (int s2 = 0; s2 < seg; ++s2) {
            const float *src = p.sums + ((size_t)bh * (p.nseg - 1) + s2) * (D * D);
#pragma unroll
            for (int i = 0; i < Cfg::SPW; ++i) {
                const int m = w + Cfg::NW * i;
                if (m < Cfg::NS) {
                    const int si = m / Cfg::TD, sj = m % Cfg::TD;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S.acc[i][r] = S.acc[i][r] * gL + src[(16 * si + 4 * gq + r) * D + 16 * sj + cl];
                }
            }
        }
    }
    S.store_copy(s, w);
    __syncthreads();
    const float gC = s.pw[C];

    const T *Add = static_cast<const T *>(p.add);
    T *Out = static_cast<T *>(p.out);
    constexpr int NTRI = Cfg::TR * (Cfg::TR + 1) / 2;
    constexpr int NOUT = Cfg::TR * Cfg::TD;

    for (int l0 = l_begin; l0 < l_end; l0 += C) {
        la_stage<T, D, C>(p, head_row, l0, s);
        __syncthreads();
        // scores: lower-triangular tiles (ti >= tj) of D_g * (A B^T)
        for (int t = w; t < NTRI; t += Cfg::NW) {
            int ti = 0;
            while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
            const int tj = t - ti * (ti + 1) / 2;
            RowFrags<T, D> fb;
            fb.template load_t<typename Ls::TR>(s.b + Ls::TR::off(16 * tj, 0));
            f32x4 acc = mma_nt_ft<typename Ls::TR, D>(zero4(), s.a + Ls::TR::off(16 * ti, 0), fb);
            const int sg = 16 * tj + cl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tau = 16 * ti + 4 * gq + r;
                const float v = tau >= sg ? acc[r] * s.pw[tau - sg] : 0.f;
                s.p[Ls::TT::off(tau, sg)] = from_f<T>(v);
            }
        }
        __syncthreads();
        // outputs, transposed: lane holds features 4gq..4gq+3 of token cl
        for (int t = w; t < NOUT; t += Cfg::NW) {
            const int tj = t % Cfg::TD, ti = t / Cfg::TD;   // feature tile, token tile
            f32x4 acc1 = zero4();
            for (int ks = 0; ks <= ti; ++ks)
                acc1 = mma16(acc1, ld_frag(s.ct + Ls::TT::off(16 * tj, 16 * ks), Ls::TT::LD),
                             ld_frag(s.p + Ls::TT::off(16 * ti, 16 * ks), Ls::TT::LD));
            RowFrags<T, D> fa;
            fa.template load_t<typename Ls::TR>(s.a + Ls::TR::off(16 * ti, 0));
            const f32x4 acc2 =
                mma_nt_ft<typename Ls::TR, D>(zero4(), s.st + Ls::TR::off(16 * tj, 0), fa);
            const int tau = 16 * ti + cl;
            const int lt = l0 + tau;
            if (lt < l_end) {
                const float sc = s.pw[tau + 1];
                const size_t row = head_row + (size_t)(p.reverse ? p.n - 1 - lt : lt);
                const size_t off = row * D + 16 * tj + 4 * gq;
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = acc1[r] + sc * acc2[r];
                if (Add) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] += to_f(Add[off + r]);
                }
                store4(Out + off, o);
            }
        }
        S.advance(s, gC, w);
        __syncthreads();
        S.store_copy(s, w);
    }
}

}  // namespace hla
