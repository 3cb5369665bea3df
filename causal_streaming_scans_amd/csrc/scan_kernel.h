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
// One workgroup per (b,h).  The up-sweep combines in place in the "e" array
// (e[i] <- e[i-s] (+) e[i]); the down-sweep writes the exclusive prefixes
// into the separate "p" array (p[i-s] <- p[i]; p[i] <- p[i] (+) e[i-s]).  The
// up-sweep skips every combine that only feeds the total (the pairs ending at
// the last slot), since an exclusive scan discards it.  Finally the caller's
// initial state, if any, is folded in front of every prefix.
//
// Each tree level runs in batches of pairs.  A batch first stages the two
// factors of every pair's cross term in LDS with coalesced vector loads (one
// round trip to memory), then one phase forms the cross terms on MFMA and
// updates every part of every pair, each element owned by one thread, so all
// of a phase's global reads are independent of each other.
#pragma once

#include "device_common.h"
#include "params.h"

namespace hla {

template <int D, int DV>
struct SumOfs {
    static constexpr int X = 0, Y = D * D, N = D * D + D * DV, y = D * D + 2 * D * DV,
                         nv = D * D + 2 * D * DV + D;
};

// Parts of one combine operand; a null part reads as zero.
struct ScanOp {
    const float *X, *Y, *N, *y, *nv;
};

__device__ __forceinline__ ScanOp scan_op(const float *base, int D, int DV) {
    return ScanOp{base, base + D * D, base + D * D + D * DV, base + D * D + 2 * D * DV,
                  base + D * D + 2 * D * DV + D};
}

__device__ __forceinline__ float rd(const float *p, int i) { return p ? p[i] : 0.f; }

// One combine of a batch: dst = A (+) B; if copy != null it also receives A
// (the down-sweep's left child).  The factor a = g^(length of B) comes from a
// separate functor, evaluated once per pair.
struct ScanPair {
    ScanOp A, B;
    float *dst;
    float *copy;
};

template <bool F32, int D, int DV>
struct ScanCfg {
    static constexpr int NT = 512, NW = NT / kWave;
    static constexpr int LDX = D + 4, LDY = DV + 4;     // fp32 rows, 16-byte aligned
    static constexpr int PAIR_FLOATS = D * LDX + D * LDY + D;
    static constexpr int PB0 = (150 * 1024) / (PAIR_FLOATS * 4);
    static constexpr int PB = PB0 < 1 ? 1 : (PB0 > 8 ? 8 : PB0);   // pairs per batch
};

// 16x16 cross-term tile from LDS: Xs rows ti*16.., Ys columns tj*16..
template <bool F32, int D, int LDX, int LDY>
__device__ __forceinline__ f32x4 cross_tile_lds(const float *Xs, const float *Ys, int ti, int tj) {
    const int l = lane_id();
    const int r = l & 15, gq = l >> 4;
    f32x4 acc = zero4();
    const float *a = Xs + (ti * 16 + r) * LDX;
    const float *b = Ys + tj * 16 + r;
    if constexpr (F32) {
#pragma unroll 4
        for (int k = 0; k < D; k += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k + gq], b[(k + gq) * LDY], acc, 0, 0, 0);
    } else if constexpr (D % 32 == 0) {
        // bf16 hi/lo split: hi*hi + hi*lo + lo*hi, one instruction shape
#pragma unroll
        for (int k = 0; k < D; k += 32) {
            bf16x8 ah, al, bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = a[k + gq * 8 + e];
                const bf16 xh = (bf16)x;
                ah[e] = xh;
                al[e] = (bf16)(x - (float)xh);
                const float y = b[(k + gq * 8 + e) * LDY];
                const bf16 yh = (bf16)y;
                bh[e] = yh;
                bl[e] = (bf16)(y - (float)yh);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int k = 0; k < D; k += 16) {
            union { bf16 h[4]; i16x4 v; } ah, al, bh, bl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = a[k + gq * 4 + e];
                const bf16 xh = (bf16)x;
                ah.h[e] = xh;
                al.h[e] = (bf16)(x - (float)xh);
                const float y = b[(k + gq * 4 + e) * LDY];
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

// dst[0:len) = a * pa + pb (when upd) and copy[0:len) = pa, as float4
// vectors; every thread issues all of its loads before any of its stores.
// len is a multiple of 4; null pa / pb read as zero.
template <int NT, int U>
__device__ __forceinline__ void lin_part(float *__restrict__ dst, float *__restrict__ copy,
                                         const float *pa, const float *pb, int len, float a,
                                         bool upd) {
    const int nv4 = len / 4;
    for (int v0 = threadIdx.x; v0 < nv4; v0 += NT * U) {
        f32x4 xa[U], xb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * NT;
            xa[u] = (v < nv4 && pa) ? reinterpret_cast<const f32x4 *>(pa)[v] : zero4();
            xb[u] = (v < nv4 && pb) ? reinterpret_cast<const f32x4 *>(pb)[v] : zero4();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * NT;
            if (v < nv4) {
                if (upd) reinterpret_cast<f32x4 *>(dst)[v] = a * xa[u] + xb[u];
                if (copy) reinterpret_cast<f32x4 *>(copy)[v] = xa[u];
            }
        }
    }
}

// Run `npair` combines (pair(j) -> ScanPair, afac(j) -> a) in batches.
// updX/updY: whether X and (Y, y) of dst are written (N and nv always are).
template <bool F32, int D, int DV, bool HLA2, typename PairFn, typename AFn>
__device__ __forceinline__ void scan_level(float *smem, float *sa, int npair, PairFn pair,
                                           AFn afac, bool updX, bool updY) {
    using G = ScanCfg<F32, D, DV>;
    using O = SumOfs<D, DV>;
    constexpr int NT = G::NT, NW = G::NW, LDX = G::LDX, LDY = G::LDY, PB = G::PB;
    constexpr int nTD = D / 16, nTV = DV / 16;
    const int w = wave_id();
    for (int j0 = 0; j0 < npair; j0 += PB) {
        const int nb = min(PB, npair - j0);
        // ---- stage the cross-term factors (Xc, Yc, yc) of every pair in the batch
        for (int b = 0; b < nb; ++b) {
            const ScanPair pr = pair(j0 + b);
            const float *Xc = HLA2 ? pr.A.X : pr.B.X;
            const float *Yc = HLA2 ? pr.B.Y : pr.A.Y;
            const float *yc = HLA2 ? pr.B.y : pr.A.y;
            float *Xs = smem + b * G::PAIR_FLOATS;
            float *Ys = Xs + D * LDX;
            float *ys = Ys + D * LDY;
            constexpr int NX4 = D * D / 4, NY4 = D * DV / 4;
            constexpr int UX = (NX4 + NT - 1) / NT, UY = (NY4 + NT - 1) / NT;
            f32x4 bx[UX], by[UY];
#pragma unroll
            for (int u = 0; u < UX; ++u) {
                const int idx = threadIdx.x + u * NT;
                bx[u] = (idx < NX4 && Xc) ? reinterpret_cast<const f32x4 *>(Xc)[idx] : zero4();
            }
#pragma unroll
            for (int u = 0; u < UY; ++u) {
                const int idx = threadIdx.x + u * NT;
                by[u] = (idx < NY4 && Yc) ? reinterpret_cast<const f32x4 *>(Yc)[idx] : zero4();
            }
            float byv = (threadIdx.x < D) ? rd(yc, threadIdx.x) : 0.f;
#pragma unroll
            for (int u = 0; u < UX; ++u) {
                const int idx = threadIdx.x + u * NT;
                if (idx < NX4) {
                    const int rr = idx / (D / 4), c = (idx % (D / 4)) * 4;
                    *reinterpret_cast<f32x4 *>(Xs + rr * LDX + c) = bx[u];
                }
            }
#pragma unroll
            for (int u = 0; u < UY; ++u) {
                const int idx = threadIdx.x + u * NT;
                if (idx < NY4) {
                    const int rr = idx / (DV / 4), c = (idx % (DV / 4)) * 4;
                    *reinterpret_cast<f32x4 *>(Ys + rr * LDY + c) = by[u];
                }
            }
            if (threadIdx.x < D) ys[threadIdx.x] = byv;
            if (threadIdx.x == 0) sa[b] = afac(j0 + b);
        }
        __syncthreads();
        // ---- N = a^2 N_A + N_B + a Xc Yc  (MFMA tiles, one wave per tile)
        for (int it = w; it < nb * nTD * nTV; it += NW) {
            const int b = it / (nTD * nTV), t = it % (nTD * nTV);
            const int ti = t / nTV, tj = t % nTV;
            const ScanPair pr = pair(j0 + b);
            float na[4], nbv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = (ti * 16 + acc_row(i)) * DV + tj * 16 + acc_col();
                na[i] = rd(pr.A.N, idx);
                nbv[i] = rd(pr.B.N, idx);
            }
            const float *Xs = smem + b * G::PAIR_FLOATS;
            const f32x4 c = cross_tile_lds<F32, D, LDX, LDY>(Xs, Xs + D * LDX, ti, tj);
            const float a = sa[b];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = (ti * 16 + acc_row(i)) * DV + tj * 16 + acc_col();
                pr.dst[O::N + idx] = a * a * na[i] + nbv[i] + a * c[i];
                if (pr.copy) pr.copy[O::N + idx] = na[i];
            }
        }
        // ---- nv = a^2 nv_A + nv_B + a Xc yc ; the linear parts X, Y, y
#pragma unroll 1
        for (int b = 0; b < nb; ++b) {
            const ScanPair pr = pair(j0 + b);
            const float a = sa[b];
            const float *Xs = smem + b * G::PAIR_FLOATS;
            const float *ys = Xs + D * LDX + D * LDY;
            for (int row = threadIdx.x; row < D; row += NT) {
                const float na = rd(pr.A.nv, row), nbv = rd(pr.B.nv, row);
                float s = 0.f;
#pragma unroll 8
                for (int c = 0; c < D; ++c) s += Xs[row * LDX + c] * ys[c];
                pr.dst[O::nv + row] = a * a * na + nbv + a * s;
                if (pr.copy) pr.copy[O::nv + row] = na;
            }
            lin_part<NT, 4>(pr.dst + O::X, pr.copy ? pr.copy + O::X : nullptr, pr.A.X, pr.B.X,
                            D * D, a, updX);
            lin_part<NT, 4>(pr.dst + O::Y, pr.copy ? pr.copy + O::Y : nullptr, pr.A.Y, pr.B.Y,
                            D * DV, a, updY);
            lin_part<NT, 1>(pr.dst + O::y, pr.copy ? pr.copy + O::y : nullptr, pr.A.y, pr.B.y, D,
                            a, updY);
        }
        __syncthreads();
    }
}

template <bool F32, int D, int DV, bool HLA2>
__global__ __launch_bounds__(512) void scan_kernel(FwdParams p) {
    constexpr int SUMF = summary_floats(D, DV);
    using G = ScanCfg<F32, D, DV>;
    constexpr int NT = G::NT;
    __shared__ alignas(16) float smem[G::PB * G::PAIR_FLOATS];
    __shared__ float sa[G::PB];
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
    auto elem = [&](float *base, int i) { return base + (size_t)i * SUMF; };

    for (size_t idx = threadIdx.x; idx < (size_t)(spad - nreal) * SUMF; idx += NT)
        E[(size_t)nreal * SUMF + idx] = 0.f;
    for (size_t idx = threadIdx.x; idx < SUMF; idx += NT) Pr[(size_t)(spad - 1) * SUMF + idx] = 0.f;
    __syncthreads();

    // ---- up-sweep: e[i] <- e[i-s] (+) e[i], i = 2s-1, 4s-1, ..., < spad-1
    for (int s = 1; s < spad; s <<= 1) {
        const int npair = spad / (2 * s) - 1;
        if (npair <= 0) continue;
        auto pair = [&](int j) {
            const int i = (j + 1) * 2 * s - 1;
            ScanPair pr;
            pr.A = scan_op(elem(E, i - s), D, DV);
            pr.B = scan_op(elem(E, i), D, DV);
            pr.dst = elem(E, i);
            pr.copy = nullptr;
            return pr;
        };
        auto afac = [&](int j) {
            const int i = (j + 1) * 2 * s - 1;
            return HLA2 ? pow_int(g, span(i - s + 1, i)) : 1.f;
        };
        scan_level<F32, D, DV, HLA2>(smem, sa, npair, pair, afac, true, true);
    }

    // ---- down-sweep: p[i-s] <- p[i];  p[i] <- p[i] (+) e[i-s]
    for (int s = spad >> 1; s >= 1; s >>= 1) {
        const int npair = spad / (2 * s);
        auto pair = [&](int j) {
            const int i = (j + 1) * 2 * s - 1;
            ScanPair pr;
            pr.A = scan_op(elem(Pr, i), D, DV);        // the prefix before the left subtree
            pr.B = scan_op(elem(E, i - s), D, DV);     // aggregate of the left subtree
            pr.dst = elem(Pr, i);
            pr.copy = elem(Pr, i - s);
            return pr;
        };
        auto afac = [&](int j) {
            const int i = (j + 1) * 2 * s - 1;
            return HLA2 ? pow_int(g, span(i - 2 * s + 1, i - s)) : 1.f;
        };
        scan_level<F32, D, DV, HLA2>(smem, sa, npair, pair, afac, true, true);
    }

    // ---- fold the caller's initial state in front of every prefix
    if (p.state_in) {
        const int STF = HLA2 ? hla2_state_floats(D, DV) : ahla_state_floats(D, DV);
        const float *st = p.state_in + (size_t)bh * STF;
        ScanOp A;
        if (HLA2) {   // (S, W, u) with C = m = 0
            A = ScanOp{st, nullptr, st + D * D, nullptr, st + D * D + D * DV};
        } else {      // (P, E, mK, nk) with M = 0
            A = ScanOp{nullptr, st, st + D * DV, st + 2 * D * DV, st + 2 * D * DV + D};
        }
        auto pair = [&](int j) {
            ScanPair pr;
            pr.A = A;
            pr.B = scan_op(elem(Pr, j), D, DV);
            pr.dst = elem(Pr, j);
            pr.copy = nullptr;
            return pr;
        };
        auto afac = [&](int j) { return HLA2 ? pow_int(g, (long)j * p.seg_len) : 1.f; };
        // HLA-2 leaves Y, y (C, m) as they are (A's are zero and the forward
        // kernel does not read them); AHLA leaves X (M).
        scan_level<F32, D, DV, HLA2>(smem, sa, p.nseg, pair, afac, HLA2, !HLA2);
    }
}

}  // namespace hla
