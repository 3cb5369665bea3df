// la_kernels.h -- chunked first-order causal linear attention on gfx950, the
// building block of the HLA-2 backward pass.
//
//   out_t = add_t + sum_{s <= t} g^(t-s) (a_t . b_s) c_s                 (plain)
//   out_t = add_t + sum_{s <= t} g^(t-s) [(a_t . b_s) c_s + (a_t . c_s) b_s]  (SYM)
//   out_t as plain, and out2_t = add2_t + sum_{s <= t} g^(t-s) (a2_t . c_s) b_s  (DUAL)
//
// and the same over the reversed sequence (s >= t, weight g^(s-t)) when
// `reverse` is set: logical token l is physical row n-1-l, so an anti-causal
// pass is the causal pass run backwards through memory.  SYM is the
// gradient of a pass whose key and value are one tensor (K in Z = LA(Q, K, K)):
// both slots in one pass, with one state S = sum w (b c^T + c b^T).  DUAL is
// two passes whose states are transposes of each other (keys and values
// swapped), which share the staged b, c and the state.
//
// The gradient of HLA-2 is a chain of such passes.  With z_t = S^K_t q_t =
// sum_{i<=t} g^(t-i) (q_t . k_i) k_i (the key read-out of page section "1. HLA
// de Segundo Orden"), the masked operator is two chained linear attentions,
// Z = LA_g(Q, K, K) and O = LA_{g^2}(Q, Z, V), and the chain rule through each
// one gives more of the same form (see hla_api.cpp).
//
// Parallel form (page section "4. Entrenamiento Paralelo mediante Escaneos
// Asociativos", first order): the state S = sum_s g^(.) b_s c_s^T is additive,
// so the sequence is cut into segments; a summary launch forms each segment's
// S from zero, and each main workgroup folds the summaries of the segments
// before its own (S <- g^len S + S_seg) and then runs its chunks.
//
// Per chunk of C tokens (one workgroup, NW = 4 waves):
//   P     = D_g * tril(A_c B_c^T)                           (C x C, in LDS, zeros above)
//   out^T = C_c^T P^T + S^T A_c^T diag(g^(tau+1)) [+ add]   (written from registers)
//   S     = g^C S + (B_c^T diag(g^(C-1-sigma))) C_c         (fp32, in registers)
// Every chunk tile is stored row-major ([token][feature]) once; products that
// contract over the tokens read their operands with the transposing LDS read
// (bf16) of device_common.h, so no transposed copy is ever written.  The
// next chunk's rows are loaded into registers while the current one computes.
#pragma once

#include <stddef.h>

#include "device_common.h"
#include "params.h"

namespace hla {

// Every array starts 16-byte aligned (the 8- and 16-byte LDS accesses need
// it; the placeholders of the arrays only SYM uses would otherwise shift
// everything after them by a few bytes, and misaligned LDS accesses cost
// several times their aligned form).
template <typename T, int D, int C, bool SYM, bool DUAL>
struct LaLds {
    using TR = LdsTile<T, D>;    // [C][D] chunk rows; [D][D] state copy St[j][i] = S[i][j]
    using TP = LdsTile<T, C>;    // [C][C] scores
    alignas(16) T a[C * TR::LD];
    alignas(16) T a2[DUAL ? C * TR::LD : 8];  // second queries (DUAL)
    alignas(16) T b[C * TR::LD];
    alignas(16) T c[C * TR::LD];
    alignas(16) T bw[C * TR::LD];            // g^(C-1-sigma) b_sigma
    alignas(16) T cw[SYM ? C * TR::LD : 8];  // g^(C-1-sigma) c_sigma (SYM)
    alignas(16) T p[C * TP::LD];
    alignas(16) T p2[SYM || DUAL ? C * TP::LD : 8];  // D_g * tril(A C^T) (SYM), D_g * tril(A2 C^T) (DUAL)
    alignas(16) T st[D * TR::LD];
    alignas(16) T ss[DUAL ? D * TR::LD : 8];  // the state itself, Ss[i][j] = S[i][j] (DUAL)
    alignas(16) float pw[C + 1];             // g^e, e = 0..C
};

template <typename T, int D, int C, bool SYM, bool DUAL>
struct LaCfg {
    using Lds = LaLds<T, D, C, SYM, DUAL>;
    static_assert(offsetof(Lds, p) % 16 == 0 && offsetof(Lds, st) % 16 == 0, "LDS tiles 16-byte aligned");
    static constexpr int NW = 4, NT = NW * kWave;
    static constexpr int TR = C / 16;          // token tiles per chunk
    static constexpr int TD = D / 16;          // feature tiles
    static constexpr int NS = TD * TD;         // state tiles
    static constexpr int SPW = (NS + NW - 1) / NW;   // state tiles per wave
    static constexpr int NSC = TR * TR;              // score tiles
    static constexpr int NOUT = TR * TD;             // output tiles
    static_assert(NSC % NW == 0 && NOUT % NW == 0, "tiles dealt evenly to the waves");
    static constexpr int blocks() {
        constexpr size_t lds = sizeof(LaLds<T, D, C, SYM, DUAL>);
        return lds <= 52 * 1024 ? 3 : (lds <= 78 * 1024 ? 2 : 1);
    }
};

// One thread's share of the a, b, c rows of a chunk, held in registers from
// the global load (a chunk ahead) to the LDS store.  Lanes run along the
// columns of a row, so one load instruction covers whole rows.  Rows past
// the end of the sequence load row 0 of the head (in bounds) and are stored
// as zeros.
template <typename T, int D, int C, int NT, bool A2>
struct LaRegs {
    static constexpr int VE = Vec16<T>::N, VPR = D / VE, NVEC = C * VPR;
    static constexpr int NV = (NVEC + NT - 1) / NT;
    uint4 ra[NV], rb[NV], rc[NV];
    uint4 ra2[A2 ? NV : 1];
    int l0;

    // WITH_A = false (segment states) skips the a rows, which only the
    // outputs read
    template <bool WITH_A = true>
    __device__ __forceinline__ void load(const LaParams &p, size_t head_row, int first) {
        l0 = first;
        const T *A = static_cast<const T *>(p.a);
        const T *B = static_cast<const T *>(p.b);
        const T *Cv = static_cast<const T *>(p.c);
        const T *A2p = static_cast<const T *>(p.a2);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + i * NT;
            const int r = idx / VPR, col = (idx % VPR) * VE;
            const int l = l0 + r;
            size_t row = head_row;
            if (idx < NVEC && l < p.n) row += (size_t)(p.reverse ? p.n - 1 - l : l);
            const size_t off = row * D + (idx < NVEC ? col : 0);
            if constexpr (WITH_A) ra[i] = *reinterpret_cast<const uint4 *>(A + off);
            if constexpr (WITH_A && A2) ra2[i] = *reinterpret_cast<const uint4 *>(A2p + off);
            rb[i] = *reinterpret_cast<const uint4 *>(B + off);
            rc[i] = *reinterpret_cast<const uint4 *>(Cv + off);
        }
    }

    // The rows' weights for the state advance are g^(cv-1-r), cv = the
    // chunk's valid rows (its last row gets g^0), so that the advance by
    // g^cv leaves the state exact after a partial last chunk too.
    template <bool WITH_A = true, bool SYM, bool DUAL>
    __device__ __forceinline__ void store(LaLds<T, D, C, SYM, DUAL> &s, int n) const {
        const int cv = n - l0 < C ? n - l0 : C;
        using TL = typename LaLds<T, D, C, SYM, DUAL>::TR;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + i * NT;
            if (idx < NVEC) {
                const int r = idx / VPR, col = (idx % VPR) * VE;
                const bool ok = l0 + r < n;
                Vec16<T> xa, xb, xc;
                // rows past the end become zeros by masking the words: a
                // select between two uint4 values kept the prefetch arrays in
                // scratch memory instead of registers
                const unsigned m = ok ? 0xffffffffu : 0u;
                uint4 ub = rb[i], uc = rc[i];
                ub.x &= m; ub.y &= m; ub.z &= m; ub.w &= m;
                uc.x &= m; uc.y &= m; uc.z &= m; uc.w &= m;
                *reinterpret_cast<uint4 *>(xb.v) = ub;
                *reinterpret_cast<uint4 *>(xc.v) = uc;
                const int o = TL::off(r, col);
                if constexpr (WITH_A) {
                    uint4 ua = ra[i];
                    ua.x &= m; ua.y &= m; ua.z &= m; ua.w &= m;
                    *reinterpret_cast<uint4 *>(xa.v) = ua;
                    store16(s.a + o, xa);
                }
                if constexpr (WITH_A && A2) {
                    static_assert(!A2 || DUAL, "second queries only in the DUAL layout");
                    uint4 ua = ra2[i];
                    ua.x &= m; ua.y &= m; ua.z &= m; ua.w &= m;
                    Vec16<T> x2;
                    *reinterpret_cast<uint4 *>(x2.v) = ua;
                    store16(s.a2 + o, x2);
                }
                store16(s.b + o, xb);
                store16(s.c + o, xc);
                const float w = r < cv ? s.pw[cv - 1 - r] : 0.f;
                Vec16<T> yb;
#pragma unroll
                for (int e = 0; e < VE; ++e) yb.v[e] = from_f<T>(to_f(xb.v[e]) * w);
                store16(s.bw + o, yb);
                if constexpr (SYM) {
                    Vec16<T> yc;
#pragma unroll
                    for (int e = 0; e < VE; ++e) yc.v[e] = from_f<T>(to_f(xc.v[e]) * w);
                    store16(s.cw + o, yc);
                }
            }
        }
    }
};

// Four consecutive values held as loaded (bf16: 8 bytes) from an early load
// to their use, converted to fp32 only there.
template <typename T> struct Raw4;
template <> struct Raw4<bf16> { uint2 u; };
template <> struct Raw4<float> { f32x4 f; };
__device__ __forceinline__ Raw4<bf16> load_raw4(const bf16 *p) { return {*reinterpret_cast<const uint2 *>(p)}; }
__device__ __forceinline__ Raw4<float> load_raw4(const float *p) { return {*reinterpret_cast<const f32x4 *>(p)}; }
__device__ __forceinline__ f32x4 raw4f(Raw4<bf16> x) {
    union { uint2 u; bf16 h[4]; } y;
    y.u = x.u;
    return f32x4{(float)y.h[0], (float)y.h[1], (float)y.h[2], (float)y.h[3]};
}
__device__ __forceinline__ f32x4 raw4f(Raw4<float> x) { return x.f; }

// acc[i][j] += sum_{k < K} M1[k][c1 + i] M2[k][c2 + j] for two row-major
// [token][feature] LDS tiles: a product over the tokens, operands read with
// the transposing LDS read (bf16) or per element (fp32).
template <typename TL, int K>
__device__ __forceinline__ f32x4 mma_tt(f32x4 acc, const bf16 *M1, int c1, const bf16 *M2, int c2) {
#pragma unroll
    for (int k = 0; k < K; k += 32)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_op8_tt<TL>(M1, k, c1), ld_op8_tt<TL>(M2, k, c2),
                                                      acc, 0, 0, 0);
    return acc;
}
template <typename TL, int K>
__device__ __forceinline__ f32x4 mma_tt(f32x4 acc, const float *M1, int c1, const float *M2, int c2) {
#pragma unroll
    for (int k = 0; k < K; k += 16) acc = mma16(acc, ld_frag_tt<TL>(M1, k, c1), ld_frag_tt<TL>(M2, k, c2));
    return acc;
}

// acc[i][j] += sum_{sigma < K} M[sigma][c1 + i] P[r2 + j][sigma]: M a
// row-major [token][feature] tile read with the transposing LDS read, P a
// row-major [token][token] score tile read along its rows.
template <typename TL, typename TPL, int K>
__device__ __forceinline__ f32x4 mma_cp(f32x4 acc, const bf16 *M, int c1, const bf16 *P, int r2) {
    const int l = lane_id();
#pragma unroll
    for (int k = 0; k < K; k += 32) {
        const bf16x8 pv = *reinterpret_cast<const bf16x8 *>(P + TPL::off(r2 + (l & 15), k + 8 * (l >> 4)));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_op8_tt<TL>(M, k, c1), pv, acc, 0, 0, 0);
    }
    return acc;
}
template <typename TL, typename TPL, int K>
__device__ __forceinline__ f32x4 mma_cp(f32x4 acc, const float *M, int c1, const float *P, int r2);

// 16-deep operand whose four k-values are consecutive in a row of an LdsTile
// matrix: lane l reads row row0 + l%16, columns col0 + 4g .. +3.
template <typename TL>
__device__ __forceinline__ Frag16<bf16> ld_frag_row(const bf16 *M, int row0, int col0) {
    const int l = lane_id();
    return Frag16<bf16>{*reinterpret_cast<const i16x4 *>(M + TL::off(row0 + (l & 15), col0 + 4 * (l >> 4)))};
}
template <typename TL>
__device__ __forceinline__ Frag16<float> ld_frag_row(const float *M, int row0, int col0) {
    const int l = lane_id();
    return Frag16<float>{*reinterpret_cast<const f32x4 *>(M + TL::off(row0 + (l & 15), col0 + 4 * (l >> 4)))};
}

template <typename TL, typename TPL, int K>
__device__ __forceinline__ f32x4 mma_cp(f32x4 acc, const float *M, int c1, const float *P, int r2) {
#pragma unroll
    for (int k = 0; k < K; k += 16) acc = mma16(acc, ld_frag_tt<TL>(M, k, c1), ld_frag_row<TPL>(P, r2, k));
    return acc;
}

// The state tiles of this wave: tile m = wave + NW*i covers S rows
// 16*(m / TD) .., columns 16*(m % TD) ..
template <typename T, int D, int C, bool SYM, bool DUAL>
struct LaState {
    using Cfg = LaCfg<T, D, C, SYM, DUAL>;
    using TL = typename LaLds<T, D, C, SYM, DUAL>::TR;
    f32x4 acc[Cfg::SPW];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < Cfg::SPW; ++i) acc[i] = zero4();
    }
    // S <- g^C S + Bw^T C (+ Cw^T B): products of the staged chunk
    __device__ __forceinline__ void advance(const LaLds<T, D, C, SYM, DUAL> &s, float gC, int w) {
#pragma unroll
        for (int i = 0; i < Cfg::SPW; ++i) {
            const int m = w + Cfg::NW * i;
            if (m < Cfg::NS) {
                const int si = m / Cfg::TD, sj = m % Cfg::TD;
                f32x4 a = acc[i];
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] *= gC;
                a = mma_tt<TL, C>(a, s.bw, 16 * si, s.c, 16 * sj);
                if constexpr (SYM) a = mma_tt<TL, C>(a, s.cw, 16 * si, s.b, 16 * sj);
                acc[i] = a;
            }
        }
    }
    // St[j][i] = S[i][j], rounded to T
    __device__ __forceinline__ void store_copy(LaLds<T, D, C, SYM, DUAL> &s, int w) const {
        const int l = lane_id(), g = l >> 4;
#pragma unroll
        for (int i = 0; i < Cfg::SPW; ++i) {
            const int m = w + Cfg::NW * i;
            if (m < Cfg::NS) {
                const int si = m / Cfg::TD, sj = m % Cfg::TD;
                store4(s.st + TL::off(16 * sj + (l & 15), 16 * si + 4 * g), acc[i]);
                if constexpr (DUAL) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s.ss[TL::off(16 * si + 4 * g + r, 16 * sj + (l & 15))] = from_f<T>(acc[i][r]);
                }
            }
        }
    }
};

// Summary of segment seg (< nseg-1): its state from zero, decayed to its end,
// into p.sums.  Grid: (nseg-1) * BH workgroups, heads fastest.
template <typename T, int D, int C, bool SYM, bool DUAL>
__device__ __forceinline__ void la_summary_body(const LaParams &p, int L, LaLds<T, D, C, SYM, DUAL> &s) {
    using Cfg = LaCfg<T, D, C, SYM, DUAL>;
    const int bh = L % p.BH, seg = L / p.BH;
    const int w = wave_id();
    const float g = p.gamma[gamma_slot(bh, p.H)];
    const size_t head_row = (size_t)bh * p.n;
    const int l_begin = seg * p.seg_len;
    const int l_end = min(p.n, l_begin + p.seg_len);
    LaRegs<T, D, C, Cfg::NT, DUAL> regs;
    regs.template load<false>(p, head_row, l_begin);
    fill_pow_table<Cfg::NT>(s.pw, C + 1, g);
    __syncthreads();
    const float gC = s.pw[C];
    LaState<T, D, C, SYM, DUAL> S;
    S.zero();
    for (int l0 = l_begin; l0 < l_end; l0 += C) {
        regs.template store<false>(s, p.n);
        if (l0 + C < l_end) regs.template load<false>(p, head_row, l0 + C);
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

template <typename T, int D, int C, bool SYM, bool DUAL>
__global__ __launch_bounds__((LaCfg<T, D, C, SYM, DUAL>::NT), (LaCfg<T, D, C, SYM, DUAL>::blocks()))
void la_summary_kernel(LaParams p) {
    __shared__ LaLds<T, D, C, SYM, DUAL> s;
    la_summary_body<T, D, C, SYM, DUAL>(p, blockIdx.x, s);
}

// The segment states of three plain passes of the same sizes in one launch:
// workgroups [i*(nseg-1)*BH, (i+1)*(nseg-1)*BH) form pass i's, so the
// three fill the compute units together instead of in turn.
struct LaParams3 {
    LaParams p[3];
};
template <typename T, int D, int C>
__global__ __launch_bounds__((LaCfg<T, D, C, false, false>::NT), (LaCfg<T, D, C, false, false>::blocks()))
void la_summary3_kernel(LaParams3 ps) {
    __shared__ LaLds<T, D, C, false, false> s;
    const int per = (ps.p[0].nseg - 1) * ps.p[0].BH;
    const int i = __builtin_amdgcn_readfirstlane(blockIdx.x / per);
    la_summary_body<T, D, C, false, false>(ps.p[i], blockIdx.x - i * per, s);
}

// Main pass over segment seg.  Grid: nseg * BH workgroups, heads fastest.
template <typename T, int D, int C, bool SYM, bool DUAL>
__global__ __launch_bounds__((LaCfg<T, D, C, SYM, DUAL>::NT), (LaCfg<T, D, C, SYM, DUAL>::blocks()))
void la_forward_kernel(LaParams p) {
    using Cfg = LaCfg<T, D, C, SYM, DUAL>;
    using Ls = LaLds<T, D, C, SYM, DUAL>;
    using TR = typename Ls::TR;
    using TP = typename Ls::TP;
    __shared__ Ls s;
    const int L = blockIdx.x;
    const int bh = L % p.BH, seg = L / p.BH;
    const int w = wave_id();
    const int l = lane_id(), gq = l >> 4, cl = l & 15;
    const float g = p.gamma[gamma_slot(bh, p.H)];
    const size_t head_row = (size_t)bh * p.n;
    const int l_begin = seg * p.seg_len;
    const int l_end = min(p.n, l_begin + p.seg_len);
    LaRegs<T, D, C, Cfg::NT, DUAL> regs;
    regs.load(p, head_row, l_begin);
    fill_pow_table<Cfg::NT>(s.pw, C + 1, g);

    // carried state: the caller's state before token 0, then the summaries
    // of the segments before this one, in order (each fold decays what is
    // already there by g^(segment length))
    LaState<T, D, C, SYM, DUAL> S;
    S.zero();
    const size_t st_stride = p.state_stride > 0 ? (size_t)p.state_stride : (size_t)(D * D);
    if (p.state_in) {
        const float *src = p.state_in + (size_t)bh * st_stride;
#pragma unroll
        for (int i = 0; i < Cfg::SPW; ++i) {
            const int m = w + Cfg::NW * i;
            if (m < Cfg::NS) {
                const int si = m / Cfg::TD, sj = m % Cfg::TD;
#pragma unroll
                for (int r = 0; r < 4; ++r) S.acc[i][r] = src[(16 * si + 4 * gq + r) * D + 16 * sj + cl];
            }
        }
    }
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

    constexpr int NO = Cfg::NOUT / Cfg::NW;   // output tiles per wave
    for (int l0 = l_begin; l0 < l_end; l0 += C) {
        const int cv = min(C, l_end - l0);   // valid rows of this chunk
        regs.store(s, p.n);
        if (l0 + C < l_end) regs.load(p, head_row, l0 + C);
        // the addends of this wave's output tiles, loaded now so that their
        // latency passes during the score phase (a row past the segment
        // reads the chunk's first row instead, in bounds and never used);
        // where Add is Out, each lane reads and later writes the same slots
        Raw4<T> ad[NO], ad2[DUAL ? NO : 1];
        if (Add || (DUAL && p.add2)) {
#pragma unroll
            for (int i = 0; i < NO; ++i) {
                const int t = w + Cfg::NW * i;
                const int tj = t % Cfg::TD, ti = t / Cfg::TD;
                const int lt = l0 + 16 * ti + cl, lr = lt < l_end ? lt : l0;
                const size_t row = head_row + (size_t)(p.reverse ? p.n - 1 - lr : lr);
                const size_t off = row * D + 16 * tj + 4 * gq;
                if (Add) ad[i] = load_raw4(Add + off);
                if constexpr (DUAL)
                    if (p.add2) ad2[i] = load_raw4(static_cast<const T *>(p.add2) + off);
            }
        }
        __syncthreads();
        // scores, transposed in registers so each lane holds four consecutive
        // sigma of one tau: every tile of D_g * (A B^T), the ones above the
        // diagonal masked to zero, so the output products below run over
        // the whole chunk with no per-tile bounds and every loop has
        // compile-time trip counts
#pragma unroll
        for (int i = 0; i < Cfg::NSC / Cfg::NW; ++i) {
            const int t = w + Cfg::NW * i;
            const int ti = t / Cfg::TR, tj = t % Cfg::TR;
            RowFrags<T, D> fa;
            fa.template load_t<TR>(s.a + 16 * ti * TR::LD);
            const int tau = 16 * ti + cl;
            f32x4 acc = mma_nt_ft<TR, D>(zero4(), s.b + 16 * tj * TR::LD, fa);
            f32x4 acc2;
            if constexpr (SYM) acc2 = mma_nt_ft<TR, D>(zero4(), s.c + 16 * tj * TR::LD, fa);
            if constexpr (DUAL) {
                RowFrags<T, D> fa2;
                fa2.template load_t<TR>(s.a2 + 16 * ti * TR::LD);
                acc2 = mma_nt_ft<TR, D>(zero4(), s.c + 16 * tj * TR::LD, fa2);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int sg = 16 * tj + 4 * gq + r;
                const float wt = tau >= sg ? s.pw[tau >= sg ? tau - sg : 0] : 0.f;
                acc[r] *= wt;
                if constexpr (SYM || DUAL) acc2[r] *= wt;
            }
            store4(s.p + TP::off(tau, 16 * tj + 4 * gq), acc);
            if constexpr (SYM || DUAL) store4(s.p2 + TP::off(tau, 16 * tj + 4 * gq), acc2);
        }
        __syncthreads();
        // outputs, transposed: lane holds features 4gq..4gq+3 of token cl
#pragma unroll
        for (int i = 0; i < NO; ++i) {
            const int t = w + Cfg::NW * i;
            const int tj = t % Cfg::TD, ti = t / Cfg::TD;   // feature tile, token tile
            f32x4 acc1 = mma_cp<TR, TP, C>(zero4(), s.c, 16 * tj, s.p, 16 * ti);
            if constexpr (SYM) acc1 = mma_cp<TR, TP, C>(acc1, s.b, 16 * tj, s.p2, 16 * ti);
            RowFrags<T, D> fa;
            fa.template load_t<TR>(s.a + 16 * ti * TR::LD);
            const f32x4 acc2 = mma_nt_ft<TR, D>(zero4(), s.st + 16 * tj * TR::LD, fa);
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
                    const f32x4 a4 = raw4f(ad[i]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] += a4[r];
                }
                store4(Out + off, o);
            }
            if constexpr (DUAL) {
                // out2 = LA(a2, c, b): scores A2 C^T, values b, state S^T
                const f32x4 b1 = mma_cp<TR, TP, C>(zero4(), s.b, 16 * tj, s.p2, 16 * ti);
                RowFrags<T, D> fa2;
                fa2.template load_t<TR>(s.a2 + 16 * ti * TR::LD);
                const f32x4 b2 = mma_nt_ft<TR, D>(zero4(), s.ss + 16 * tj * TR::LD, fa2);
                if (lt < l_end) {
                    const float sc = s.pw[tau + 1];
                    const size_t row = head_row + (size_t)(p.reverse ? p.n - 1 - lt : lt);
                    f32x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = b1[r] + sc * b2[r];
                    const size_t off = row * D + 16 * tj + 4 * gq;
                    if (p.add2) {
                        const f32x4 a4 = raw4f(ad2[i]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) o[r] += a4[r];
                    }
                    store4(static_cast<T *>(p.out2) + off, o);
                }
            }
        }
        S.advance(s, cv == C ? gC : s.pw[cv], w);
        __syncthreads();
        S.store_copy(s, w);
    }
    if (seg == p.nseg - 1) {
        // the state after token n-1
        for (float *base : {p.state_out, p.state_out2}) {
            if (!base) continue;
            float *dst = base + (size_t)bh * st_stride;
#pragma unroll
            for (int i = 0; i < Cfg::SPW; ++i) {
                const int m = w + Cfg::NW * i;
                if (m < Cfg::NS) {
                    const int si = m / Cfg::TD, sj = m % Cfg::TD;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dst[(16 * si + 4 * gq + r) * D + 16 * sj + cl] = S.acc[i][r];
                }
            }
        }
    }
}

}  // namespace hla

namespace hla {

// ------------------------------------------------ ratio form of the backward
//
// With o = num / den (num = LA_{g^2}(Q, Z, V), den its v == 1 sum), the
// gradient is that of num with the upstream gradient dO / den, plus the
// terms of den with e_t = -(dO_t . o_t) / den_t.  The ones column of den is
// carried by a tensor whose rows are the unit vector (1, 0, ..., 0) (ONE1),
// and e by one whose rows are (e_t, 0, ..., 0) (E1), so that LA passes of
// the same kernels form u_t = sum_j g^(2(t-j)) z_j = LA(ONE1, ONE1, Z)_t and
// r_j = sum_{t>=j} g^(2(t-j)) e_t q_t = RLA(ONE1, E1, Q)_j.

// rows of ONE1 (a unit first column) into out: [rows][D]
template <typename T, int D>
__global__ __launch_bounds__(256) void unit_column_kernel(T *out, long rows) {
    const long total = rows * D;
    const long stride = (long)gridDim.x * blockDim.x;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride)
        out[i] = from_f<T>(i % D == 0 ? 1.f : 0.f);
}

// Row-wise division of the third-order ratio form: out[t][:] = num[t][:] /
// den[t][0], with num and den fp32 [rows][D] and out of element type TO.
// Four consecutive values per thread; a zero den gives IEEE inf / NaN.
template <typename TO, int D>
__global__ __launch_bounds__(256) void divide_rows_kernel(const float *num, const float *den,
                                                          TO *out, long rows) {
    constexpr int Q4 = D / 4;
    const long total = rows * Q4;
    const long stride = (long)gridDim.x * blockDim.x;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const long row = i / Q4;
        const f32x4 x = reinterpret_cast<const f32x4 *>(num)[i];
        const float dn = den[(size_t)row * D];
        store4(out + 4 * i, f32x4{x[0] / dn, x[1] / dn, x[2] / dn, x[3] / dn});
    }
}

// One wave per row t:
//   den = q . u,  o = num / den,  g = dO / den,  e = -(dO . o) / den;
//   writes g into G, (e, 0, ..., 0) into E1, and e u into dq.
template <typename T, int D>
__global__ __launch_bounds__(256) void ratio_prep_kernel(RatioPrepParams p) {
    constexpr int PER = (D + kWave - 1) / kWave;
    const long row = (long)blockIdx.x * (256 / kWave) + wave_id();
    if (row >= p.rows) return;
    const int l = lane_id();
    const size_t base = (size_t)row * D;
    const T *q = static_cast<const T *>(p.q) + base;
    const T *u = static_cast<const T *>(p.u) + base;
    const T *num = static_cast<const T *>(p.num) + base;
    const T *dout = static_cast<const T *>(p.dout) + base;
    float qv[PER], uv[PER], nv[PER], dv[PER];
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int c = l + kWave * j;
        const bool ok = c < D;
        qv[j] = ok ? to_f(q[c]) : 0.f;
        uv[j] = ok ? to_f(u[c]) : 0.f;
        nv[j] = ok ? to_f(num[c]) : 0.f;
        dv[j] = ok ? to_f(dout[c]) : 0.f;
        den += qv[j] * uv[j];
    }
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) den += __shfl_xor(den, m, kWave);
    const float inv = 1.f / den;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) dot += dv[j] * nv[j] * inv;
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) dot += __shfl_xor(dot, m, kWave);
    const float e = -dot * inv;
    T *G = static_cast<T *>(p.g) + base;
    T *E1 = static_cast<T *>(p.e1) + base;
    T *dq = static_cast<T *>(p.dq) + base;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int c = l + kWave * j;
        if (c < D) {
            G[c] = from_f<T>(dv[j] * inv);
            E1[c] = from_f<T>(c == 0 ? e : 0.f);
            dq[c] = from_f<T>(e * uv[j]);
        }
    }
}

// 16 bytes of a row as floats: 8 bf16 or 4 fp32 values.
template <typename T> struct Row16;
template <> struct Row16<bf16> {
    static constexpr int N = 8;
    float x[8];
    __device__ __forceinline__ void load(const bf16 *p) {
        const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
    }
};
template <> struct Row16<float> {
    static constexpr int N = 4;
    float x[4];
    __device__ __forceinline__ void load(const float *p) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = v[j];
    }
};

// Decay gradient, first step: workgroup (x, bh) sums the weighted row terms
// of DecayGradParams over rows x*RPB + i*nblk*RPB + ...  Each row is read by
// D/N lanes with one 16-byte load per tensor (N values each); the row term is
// formed in fp32 and weighted and summed in fp64.  One partial per
// workgroup, no atomics.
template <typename T, int D>
__global__ __launch_bounds__(256) void decay_grad_rows_kernel(DecayGradParams p) {
    using R = Row16<T>;
    constexpr int LPR = D / R::N;           // lanes per row
    constexpr int RPW = kWave / LPR;        // rows per wave and step
    constexpr int RPB = RPW * (256 / kWave);
    static_assert(D % R::N == 0 && kWave % LPR == 0, "row split");
    const int bh = blockIdx.y;
    const int l = lane_id(), w = wave_id();
    const int sub = l / LPR, part = l % LPR;
    const double mid = 0.5 * (double)(p.n - 1);
    const size_t head = (size_t)bh * p.n * D;
    const T *Q = static_cast<const T *>(p.q) + head, *K = static_cast<const T *>(p.k) + head;
    const T *Zt = static_cast<const T *>(p.z) + head, *dQ = static_cast<const T *>(p.dq) + head;
    const T *dK = static_cast<const T *>(p.dk) + head, *dZ = static_cast<const T *>(p.dz) + head;
    double acc = 0.0;
    // the loop bound is uniform over the wave; rows past n contribute zero
    for (long t0 = (long)blockIdx.x * RPB + w * RPW; t0 < p.n; t0 += (long)p.nblk * RPB) {
        const long t = t0 + sub;
        float s = 0.f;
        if (t < p.n) {
            const size_t off = (size_t)t * D + part * R::N;
            R q, dq, z, dz, k, dk;
            q.load(Q + off);
            dq.load(dQ + off);
            z.load(Zt + off);
            dz.load(dZ + off);
            k.load(K + off);
            dk.load(dK + off);
#pragma unroll
            for (int j = 0; j < R::N; ++j)
                s += 2.f * q.x[j] * dq.x[j] - 3.f * z.x[j] * dz.x[j] - 0.5f * k.x[j] * dk.x[j];
        }
#pragma unroll
        for (int m = LPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, kWave);
        if (part == 0 && t < p.n) acc += ((double)t - mid) * (double)s;
    }
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, kWave);
    __shared__ double wsum[256 / kWave];
    if (l == 0) wsum[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
#pragma unroll
        for (int i = 0; i < 256 / kWave; ++i) tot += wsum[i];
        p.partial[(size_t)bh * p.nblk + blockIdx.x] = tot;
    }
}

// Decay gradient, second step: one wave per head h.  Lane i sums the
// partials i, i + 64, ... of heads b*H + h (b in order), the lanes are then
// combined by a fixed butterfly, and dgamma[h] = sum / g_h.
__global__ __launch_bounds__(kWave) void decay_grad_final_kernel(DecayGradParams p) {
    const int h = blockIdx.x, l = lane_id();
    const int B = p.BH / p.H;
    double tot = 0.0;
    for (int b = 0; b < B; ++b) {
        const double *row = p.partial + (size_t)(b * p.H + h) * p.nblk;
        for (int x = l; x < p.nblk; x += kWave) tot += row[x];
    }
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) tot += __shfl_xor(tot, m, kWave);
    if (l == 0) p.dgamma[h] = (float)(tot / (double)p.gamma[gamma_slot(h, p.H)]);
}

}  // namespace hla

namespace hla {

// bf16 <-> fp32 copies of whole tensors (the ratio backward keeps its passes
// in fp32, see hla_api.cpp); count is a multiple of 4
__global__ __launch_bounds__(256) void widen_kernel(const bf16 *src, float *dst, long count4) {
    const long stride = (long)gridDim.x * blockDim.x;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < count4; i += stride) {
        union { uint2 u; bf16 h[4]; } x;
        x.u = reinterpret_cast<const uint2 *>(src)[i];
        reinterpret_cast<f32x4 *>(dst)[i] = f32x4{(float)x.h[0], (float)x.h[1], (float)x.h[2], (float)x.h[3]};
    }
}
__global__ __launch_bounds__(256) void narrow_kernel(const float *src, bf16 *dst, long count4) {
    const long stride = (long)gridDim.x * blockDim.x;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < count4; i += stride)
        store4(dst + 4 * i, reinterpret_cast<const f32x4 *>(src)[i]);
}

}  // namespace hla
