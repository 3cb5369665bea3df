// ahla_kernels.h -- chunked asymmetric HLA (AHLA) on gfx950: segment-summary
// kernel and forward kernel.
//
// Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
// gist.science/es/paper/2510.27258, section "2. Atencion Lineal de Orden
// Superior Asimetrica (AHLA)": the operator Q (K^T Q)(K^T V), masked, with the
// streaming summaries P^KV, m^K, E and n.
//
// Chunk form (derived from those summaries): y_t = P_t^T q_t is causal linear
// attention, and o_t = q_t^T E_t with E_t = g E_{t-1} + k_t y_t^T.  With a
// decay g every summary decays by g per token ("Contribuciones Clave", item
// 2: masked operators with exponential decay; g = 1 without), so the term
// A[t,i] A[i,j] v_j of o_t carries g^(t-j).  For a chunk with carried
// (P0, E0, mK0, nk0), in-chunk positions tau and L = D_g * tril(Q K^T):
//     Y  = diag(g^(tau+1)) Q P0 + L V       y1 = diag(g^(tau+1)) Q mK0 + L 1
//     O  = diag(g^(tau+1)) Q E0 + L Y       den = diag(g^(tau+1)) Q nk0 + L y1
//     P0 <- g^c P0 + K^T diag(g^(c-1-tau)) V ; E0 likewise with Y;
//     mK0, nk0 likewise with the v == 1 column and y1
// The summary kernel runs this from zero over one segment and also forms
// M = sum_t k_t q_t^T (undecayed), the factor of the segment combine's cross
// term a M_B P_A (a = g^(tokens of B)).
//
// Work split and LDS layout as for HLA-2: wave (r, cg) owns row tile r and
// column tiles cg, cg + NCG, ...; chunk tiles sit in LDS row-major and every
// product over the tokens reads them through the transposing LDS read.  The
// transposed scores L^T = K Q^T stay in registers and serve as the B operand
// of V^T L^T (for Y^T) and of Y^T L^T (for O^T).  Y^T's accumulator holds
// four consecutive features of one token, so Y goes to LDS row-major with
// one 8-byte store per tile.  P, E are widened by the mK / nk column, and
// the products that need the matching column of V or Y take a ones column
// tile (a constant operand fragment) or the y1 column tile (its own small
// LDS tile): y1 = Q mK0 + L 1, the ratio denominator Q nk0 + L y1,
// mK += K^T 1 and nk += K^T y1.  Chunk tiles and state copies use the
// LdsTile layout (swizzled 128-byte rows for bf16 with 64 columns).
#pragma once

#include "chunk_common.h"
#include "hla2_kernels.h"

namespace hla {

template <typename T, int D, int DV, int C>
struct AhlaCfg {
    static constexpr int NPOW = C + 2;        // g^e, e = 0 .. C+1
    using WS = WaveShape<C, D>;
    static constexpr int RT = WS::RT, NCG = WS::NCG, NW = WS::NW, NT = WS::NT;
    static constexpr int DVX = DV + 16;       // P, E widened by the mK / nk column tile
    using TK = LdsTile<T, D>;                 // Q, K chunk rows; the state copies Pt, Et
    using TV = LdsTile<T, DV>;                // V, Y chunk rows
    using TY1 = PadTile<T, 16>;               // the y1 column tile of Y
    static constexpr int nTD = D / 16, nTV = DV / 16;
    static constexpr int OJ = (nTV + NCG - 1) / NCG;      // O^T tiles per wave
    static constexpr int YJ = (nTV + 1 + NCG - 1) / NCG;  // Y^T tiles per wave, widened
    static constexpr int UJ = (nTD + NW - 1) / NW;        // mK / nk column tiles per wave
    using PBk = TileBlocks<nTD, nTV, NW>;   // ownership of P, E tiles
    using MBk = TileBlocks<nTD, nTD, NW>;   // ownership of M tiles
    static constexpr int SUMF = summary_floats(D, DV);
    static constexpr int STF = ahla_state_floats(D, DV);
    static_assert(D % 16 == 0 && DV % 16 == 0 && C % 16 == 0, "tile multiples");
};

template <typename T, int D, int DV, int C, bool DECAY>
struct AhlaFwdSmem {
    using G = AhlaCfg<T, D, DV, C>;
    alignas(16) T K[C * G::TK::LD];
    alignas(16) T Kw[DECAY ? C * G::TK::LD : 8];   // rows weighted by g^(c-1-tau)
    alignas(16) T V[C * G::TV::LD];
    alignas(16) T Y[C * G::TV::LD];
    alignas(16) T Y1[C * G::TY1::LD];      // column 0 = y1
    alignas(16) T Pt[G::DVX * G::TK::LD];  // Pt[j][i] = P0[i][j]; row DV = mK0
    alignas(16) T Et[G::DVX * G::TK::LD];  // Et[j][i] = E0[i][j]; row DV = nk0
    // each wave's 16 output rows on their way out (one wave per row tile)
    alignas(16) T Ot[G::NCG == 1 && sizeof(T) == 2 ? G::RT * 16 * G::TV::LD : 8];
    float gp[DECAY ? G::NPOW : 1];
};

template <typename T, int D, int DV, int C, bool DECAY>
using AhlaFwdLds = LdsWithScratch<AhlaFwdSmem<T, D, DV, C, DECAY>, CrossLds<D, DV>::FLOATS>;

template <typename T, int D, int DV, int C, bool DECAY>
struct AhlaSumSmem {
    using G = AhlaCfg<T, D, DV, C>;
    alignas(16) T Q[C * G::TK::LD];
    alignas(16) T K[C * G::TK::LD];
    alignas(16) T Kw[DECAY ? C * G::TK::LD : 8];
    alignas(16) T V[C * G::TV::LD];
    alignas(16) T Y[C * G::TV::LD];
    alignas(16) T Y1[C * G::TY1::LD];
    alignas(16) T Pt[G::DVX * G::TK::LD];
    float gp[DECAY ? G::NPOW : 1];
};

// Built for at most two workgroups per CU: the register budget of a third
// (168 VGPRs) makes both kernels spill at chunk 64.
template <typename T, int D, int DV, int C, bool DECAY>
constexpr int ahla_fwd_blocks() {
    const int b = hla_min_blocks<AhlaCfg<T, D, DV, C>::NT, (int)sizeof(AhlaFwdLds<T, D, DV, C, DECAY>)>();
    return b > 2 ? 2 : b;
}
template <typename T, int D, int DV, int C, bool DECAY>
constexpr int ahla_sum_blocks() {
    const int b = hla_min_blocks<AhlaCfg<T, D, DV, C>::NT, (int)sizeof(AhlaSumSmem<T, D, DV, C, DECAY>)>();
    return C >= 64 && b > 2 ? 2 : b;
}

// Y^T tiles of row tile R: Y = diag(g^(tau+1)) Q P0 + L V, and the y1 tile
// (the same with mK0 and the v == 1 column, in Y1) when `wide`; stored
// row-major after every product.
template <typename T, int D, int DV, int R, int NCG, int YJ, typename G, bool DECAY>
__device__ __forceinline__ void ahla_y_tiles(const RowFrags<T, D> &qf, const Frag16<T> (&Lf)[R + 1],
                                             const T *Pt, const T *V, T *Y, T *Y1, int cg, int tau,
                                             bool wide, const float *gp) {
    using TK = typename G::TK;
    using TV = typename G::TV;
    constexpr int nTV = DV / 16;
    const int g4 = (lane_id() >> 4) << 2;
    f32x4 y[YJ];
#pragma unroll
    for (int jj = 0; jj < YJ; ++jj) {
        const int jv = cg + jj * NCG;
        y[jj] = zero4();
        if (jv < nTV || (wide && jv == nTV)) {
            f32x4 yq = mma_nt_ft<TK>(zero4(), Pt + 16 * jv * TK::LD, qf);
            if (DECAY) yq *= gp[tau + 1];
            f32x4 yc = zero4();
#pragma unroll
            for (int s = 0; s <= R; ++s)
                yc = mma16(yc, jv < nTV ? ld_frag_tt<TV>(V, 16 * s, 16 * jv) : ones_frag<T>(), Lf[s]);
            y[jj] = yq + yc;
        }
    }
#pragma unroll
    for (int jj = 0; jj < YJ; ++jj) {
        const int jv = cg + jj * NCG;
        if (jv < nTV) store4(Y + TV::off(tau, 16 * jv + g4), y[jj]);
        else if (wide && jv == nTV) store4(Y1 + G::TY1::off(tau, g4), y[jj]);
    }
}

// YO: also write the first pass's rows y_t = P_t^T q_t (Y = LA_g(Q, K, V))
// to p.z_out.
template <typename T, int D, int DV, int C, bool DECAY, bool YO = false>
__global__ __launch_bounds__((AhlaCfg<T, D, DV, C>::NT), (ahla_fwd_blocks<T, D, DV, C, DECAY>()))
void ahla_forward_kernel(FwdParams p) {
    using G = AhlaCfg<T, D, DV, C>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    constexpr int nTD = G::nTD, nTV = G::nTV;
    using TK = typename G::TK;
    using TV = typename G::TV;
    using TY1 = typename G::TY1;
    __shared__ AhlaFwdLds<T, D, DV, C, DECAY> lds;
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
    // u-type summaries always carried and the ratio's products always
    // formed, so the chunk loop has no wave-uniform branches (as in the
    // HLA-2 forward, where such branches gave run-to-run errors)
    constexpr bool need_u = true;
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * p.n * DV;
    // one wave per row tile: output rows staged in LDS, stored whole
    constexpr bool ROWS_OUT = NCG == 1 && sizeof(T) == 2;
    const __amdgpu_buffer_rsrc_t orsrc = rows_rsrc(o + (size_t)t_begin * DV, t_end - t_begin, DV);
    T *yo = YO ? static_cast<T *>(p.z_out) + ((size_t)bh * p.n + t_begin) * DV : nullptr;
    const __amdgpu_buffer_rsrc_t yrsrc = rows_rsrc(yo, YO ? t_end - t_begin : 0, DV);

    // the next chunk's data in registers: K, V for LDS; this wave's Q rows
    ChunkRegs<T, C, D, NT> rk;
    ChunkRegs<T, C, DV, NT> rv;
    RowFrags<T, D> qn;
    auto load_chunk = [&](int c, int valid) {
        const int tv = valid - 16 * r;
        qn.load_rows_g(q + (size_t)(c + (tv > 0 ? 16 * r : 0)) * D, D, tv > 0 ? tv : 0);
        rk.load(k + (size_t)c * D, valid);
        rv.load(v + (size_t)c * DV, valid);
    };

    // carried state at the start of this segment: the caller's state (or
    // zero), then the up-sweep nodes covering segments 0 .. seg-1
    const float *P0 = nullptr, *E0 = nullptr, *mK0 = nullptr, *nk0 = nullptr;
    if (p.state_in) {
        const float *e = p.state_in + (size_t)bh * G::STF;
        P0 = e;
        E0 = e + D * DV;
        mK0 = e + 2 * D * DV;
        nk0 = mK0 + D;
    }
    using PBk = typename G::PBk;
    using O = SumOfs<D, DV>;
    f32x4 accP[PBk::PB][PBk::BR][PBk::BR], accE[PBk::PB][PBk::BR][PBk::BR];
    f32x4 accMK[G::UJ], accNK[G::UJ];
    for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = (16 * ti + g4 + i) * DV + 16 * tv + col;
            accP[pb][x][y][i] = P0 ? P0[idx] : 0.f;
            accE[pb][x][y][i] = E0 ? E0[idx] : 0.f;
        }
    });
    // mK, nk as column DV of the widened P, E (the other 15 columns zero)
    for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            accMK[j][i] = (mK0 && col == 0) ? mK0[16 * ti + g4 + i] : 0.f;
            accNK[j][i] = (nk0 && col == 0) ? nk0[16 * ti + g4 + i] : 0.f;
        }
    });
    if (seg > 0) {
        // fold node B (later) into the running state A, a = g^(tokens of B):
        // E <- a E + E_B + a M_B P, nk <- a nk + nk_B + a M_B mK,
        // P <- a P + P_B, mK <- a mK + mK_B; the node's M and the old widened
        // [P | mK] are staged in LDS (fp32)
        using L = CrossLds<D, DV>;  // fold: whole right factor
        float *Ms = lds.f, *Ps = lds.f + D * L::LDA;
        int done = 0;
        while (done < seg) {
            // the next node: a leaf, or the largest up-sweep node left
            const int b = p.leaf_fold ? 0 : 31 - __builtin_clz(seg - done);
            const float *e = p.ws + node_offset(bh, b, done >> b, p.BH, p.nreal, G::SUMF);
            const float a = DECAY ? pow_int(g, (long)p.seg_len << b) : 1.f;
            // with no caller state the first node folds into zero: no cross terms
            const bool cross = p.state_in != nullptr || done > 0;
            // The node's linear parts: with d <= 64 they are loaded into
            // registers ahead of the staging, so every global load of the node
            // is in flight at once (larger heads have no registers to spare)
            constexpr bool PRE = D <= 64;
            float ne[PBk::PB][PBk::BR][PBk::BR][PRE ? 4 : 1], np[PBk::PB][PBk::BR][PBk::BR][PRE ? 4 : 1];
            float nn[G::UJ][PRE ? 4 : 1], nm[G::UJ][PRE ? 4 : 1];
            auto ev = [&](int ofs, int ti, int tv, int i) { return e[ofs + (16 * ti + g4 + i) * DV + 16 * tv + col]; };
            auto vv = [&](int ofs, int ti, int i) { return col == 0 ? e[ofs + 16 * ti + g4 + i] : 0.f; };
            if constexpr (PRE) {
                for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ne[pb][x][y][i] = ev(O::N, ti, tv, i);
                        np[pb][x][y][i] = ev(O::Y, ti, tv, i);
                    }
                });
                for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        nn[j][i] = vv(O::nv, ti, i);
                        nm[j][i] = vv(O::y, ti, i);
                    }
                });
            }
            if (cross) {
                for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Ps[(16 * ti + g4 + i) * L::LDB + 16 * tv + col] = accP[pb][x][y][i];
                });
                for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) Ps[(16 * ti + g4 + i) * L::LDB + DV + col] = accMK[j][i];
                });
                stage_f32<D, D, NT>(Ms, L::LDA, e + O::X, D);
            }
            // the linear terms now (the old P, mK are already staged); the
            // cross terms once the staging has landed
            for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accE[pb][x][y][i] = a * accE[pb][x][y][i] + (PRE ? ne[pb][x][y][PRE ? i : 0] : ev(O::N, ti, tv, i));
                    accP[pb][x][y][i] = a * accP[pb][x][y][i] + (PRE ? np[pb][x][y][PRE ? i : 0] : ev(O::Y, ti, tv, i));
                }
            });
            for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accNK[j][i] = a * accNK[j][i] + (PRE ? nn[j][PRE ? i : 0] : vv(O::nv, ti, i));
                    accMK[j][i] = a * accMK[j][i] + (PRE ? nm[j][PRE ? i : 0] : vv(O::y, ti, i));
                }
            });
            if (cross) {
                __syncthreads();
                for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
                    accE[pb][x][y] += a * tile_ab_f32<D>(Ms + 16 * ti * L::LDA, L::LDA, Ps + 16 * tv, L::LDB);
                });
                for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
                    accNK[j] += a * tile_ab_f32<D>(Ms + 16 * ti * L::LDA, L::LDA, Ps + DV, L::LDB);
                });
                __syncthreads();
            }
            done += 1 << b;
        }
    }
    for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
        store4(sm.Pt + TK::off(16 * tv + col, 16 * ti + g4), accP[pb][x][y]);
        store4(sm.Et + TK::off(16 * tv + col, 16 * ti + g4), accE[pb][x][y]);
    });
    for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
        store4(sm.Pt + TK::off(DV + col, 16 * ti + g4), accMK[j]);
        store4(sm.Et + TK::off(DV + col, 16 * ti + g4), accNK[j]);
    });
    if (DECAY) fill_pow_table<NT>(sm.gp, G::NPOW, g);

    int c0 = t_begin;
    int cv = min(C, t_end - c0);
    load_chunk(c0, cv);

    while (c0 < t_end) {
        __syncthreads();
        rk.template store_tile<TK>(sm.K);
        if (DECAY) rk.template store_tile_w<TK>(sm.Kw, sm.gp, cv - 1);
        rv.template store_tile<TV>(sm.V);
        RowFrags<T, D> qf = qn;
        qf.mask_rows(cv - 16 * r);
        const int n0 = c0 + C;
        const int ncv = min(C, t_end - n0);
        if (n0 < t_end) load_chunk(n0, ncv);
        __syncthreads();

        with_row_tile<RT>(r, [&](auto rt) {
            constexpr int R = decltype(rt)::value;
            const int tau = 16 * R + col;
            Frag16<T> Lf[R + 1];
            scores_t<T, D, R, TK, DECAY>(Lf, sm.K, qf, tau, DECAY ? sm.gp : nullptr, 1);
            ahla_y_tiles<T, D, DV, R, NCG, G::YJ, G, DECAY>(qf, Lf, sm.Pt, sm.V, sm.Y, sm.Y1, cg, tau,
                                                            need_u, DECAY ? sm.gp : nullptr);
            // carried part of the output and of its denominator (row DV)
            f32x4 accO[G::OJ];
#pragma unroll
            for (int jj = 0; jj < G::OJ; ++jj) {
                const int jv = cg + jj * NCG;
                accO[jj] = zero4();
                if (jv < nTV) {
                    accO[jj] = mma_nt_ft<TK>(zero4(), sm.Et + 16 * jv * TK::LD, qf);
                    if (DECAY) accO[jj] *= sm.gp[tau + 1];
                }
            }
            f32x4 accD = mma_nt_ft<TK>(zero4(), sm.Et + DV * TK::LD, qf);
            if (DECAY) accD *= sm.gp[tau + 1];
            __syncthreads();

            // O^T += Y^T L^T ; den = q . nk0 + sum_sigma L[tau][sigma] y1[sigma]
            f32x4 dc = zero4();
#pragma unroll
            for (int s = 0; s <= R; ++s) dc = mma16(dc, ld_frag_tt<TY1>(sm.Y1, 16 * s, 0), Lf[s]);
            const float den = __shfl(accD[0] + dc[0], col);
            const float rden = ratio ? 1.f / den : 1.f;
#pragma unroll
            for (int jj = 0; jj < G::OJ; ++jj) {
                const int jv = cg + jj * NCG;
                if (jv < nTV) {
                    f32x4 oc = zero4();
#pragma unroll
                    for (int s = 0; s <= R; ++s)
                        oc = mma16(oc, ld_frag_tt<TV>(sm.Y, 16 * s, 16 * jv), Lf[s]);
                    const f32x4 ov = (accO[jj] + oc) * rden;
                    if constexpr (ROWS_OUT) store4(sm.Ot + (R * 16) * TV::LD + TV::off(col, 16 * jv + g4), ov);
                    else store4_row<T>(orsrc, ((c0 - t_begin + tau) * DV + 16 * jv + g4) * (int)sizeof(T), ov);
                }
            }
            if constexpr (ROWS_OUT)
                store_rows_out<T, TV, DV>(sm.Ot + (R * 16) * TV::LD, orsrc, c0 - t_begin + 16 * R);
            // the rows of Y, whole since the barrier above: this wave's rows,
            // its column group's share of them
            if constexpr (YO)
                copy_rows_out<T, TV, DV / NCG, DV>(sm.Y, yrsrc, 16 * R, c0 - t_begin + 16 * R, cg * (DV / NCG));
        });
        // advance the state: P0 <- g^c P0 + Kw^T V, E0 likewise with Y, mK0
        // with the ones column, nk0 with y1 (Kw: K rows weighted by
        // g^(c-1-tau)); all products first, then the T-typed copies
        const T *KA = DECAY ? sm.Kw : sm.K;
        const float gc = DECAY ? sm.gp[cv] : 1.f;
        for_blocks<PBk, NW>(w, [&](int pb, int ti0, int tv0) {
            if (DECAY) {
#pragma unroll
                for (int x = 0; x < PBk::BR * PBk::BR; ++x) {
                    (&accP[pb][0][0])[x] *= gc;
                    (&accE[pb][0][0])[x] *= gc;
                }
            }
            mma_tn_grp<PBk::BR, PBk::BR, C, TK, TV, false>(&accP[pb][0][0], KA, 16 * ti0, sm.V, 16 * tv0);
            mma_tn_grp<PBk::BR, PBk::BR, C, TK, TV, false>(&accE[pb][0][0], KA, 16 * ti0, sm.Y, 16 * tv0);
        });
        if (need_u) {
            for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
                if (DECAY) {
                    accMK[j] *= gc;
                    accNK[j] *= gc;
                }
                mma_tn_grp<1, 1, C, TK, TV, true>(&accMK[j], KA, 16 * ti, sm.V, 0);
                mma_tn_grp<1, 1, C, TK, TY1, false>(&accNK[j], KA, 16 * ti, sm.Y1, 0);
            });
        }
        for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
            const int oo = TK::off(16 * tv + col, 16 * ti + g4);
            store4(sm.Pt + oo, accP[pb][x][y]);
            store4(sm.Et + oo, accE[pb][x][y]);
        });
        if (need_u) {
            for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
                store4(sm.Pt + TK::off(DV + col, 16 * ti + g4), accMK[j]);
                store4(sm.Et + TK::off(DV + col, 16 * ti + g4), accNK[j]);
            });
        }
        c0 = n0;
        cv = ncv;
    }

    if (p.state_out && last) {
        float *so = p.state_out + (size_t)bh * G::STF;
        for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = (16 * ti + g4 + i) * DV + 16 * tv + col;
                so[idx] = accP[pb][x][y][i];
                so[D * DV + idx] = accE[pb][x][y][i];
            }
        });
        for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
            if (col == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    so[2 * D * DV + 16 * ti + g4 + i] = accMK[j][i];
                    so[2 * D * DV + D + 16 * ti + g4 + i] = accNK[j][i];
                }
            }
        });
    }
}

template <typename T, int D, int DV, int C, bool DECAY>
__global__ __launch_bounds__((AhlaCfg<T, D, DV, C>::NT), (ahla_sum_blocks<T, D, DV, C, DECAY>()))
void ahla_summary_kernel(FwdParams p) {
    using G = AhlaCfg<T, D, DV, C>;
    constexpr int NT = G::NT, NW = G::NW, NCG = G::NCG, RT = G::RT;
    constexpr int nTD = G::nTD;
    using TK = typename G::TK;
    using TV = typename G::TV;
    using TY1 = typename G::TY1;
    __shared__ AhlaSumSmem<T, D, DV, C, DECAY> sm;

    const int seg = blockIdx.x, bh = blockIdx.y;
    const float g = DECAY ? p.gamma[gamma_slot(bh, p.H)] : 1.f;
    const int w = wave_id();
    const int r = w / NCG, cg = w % NCG;
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;

    using PBk = typename G::PBk;
    using MBk = typename G::MBk;
    f32x4 accP[PBk::PB][PBk::BR][PBk::BR], accE[PBk::PB][PBk::BR][PBk::BR];
    f32x4 accM[MBk::PB][MBk::BR][MBk::BR], accMK[G::UJ], accNK[G::UJ];
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
#pragma unroll
    for (int j = 0; j < G::UJ; ++j) {
        accMK[j] = zero4();
        accNK[j] = zero4();
    }
    for (int i = threadIdx.x; i < G::DVX * TK::LD; i += NT) sm.Pt[i] = from_f<T>(0.f);
    if (DECAY) fill_pow_table<NT>(sm.gp, G::NPOW, g);

    ChunkRegs<T, C, D, NT> rq, rk;
    ChunkRegs<T, C, DV, NT> rv;
    int c0 = t_begin;
    int cv = min(C, t_end - c0);
    rq.load(q + (size_t)c0 * D, cv);
    rk.load(k + (size_t)c0 * D, cv);
    rv.load(v + (size_t)c0 * DV, cv);

    while (c0 < t_end) {
        __syncthreads();
        rq.template store_tile<TK>(sm.Q);
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

        RowFrags<T, D> qf;
        qf.template load_t<TK>(sm.Q + 16 * r * TK::LD);
        with_row_tile<RT>(r, [&](auto rt) {
            constexpr int R = decltype(rt)::value;
            const int tau = 16 * R + col;
            Frag16<T> Lf[R + 1];
            scores_t<T, D, R, TK, DECAY>(Lf, sm.K, qf, tau, DECAY ? sm.gp : nullptr, 1);
            ahla_y_tiles<T, D, DV, R, NCG, G::YJ, G, DECAY>(qf, Lf, sm.Pt, sm.V, sm.Y, sm.Y1, cg, tau,
                                                            true, DECAY ? sm.gp : nullptr);
        });
        __syncthreads();

        // P <- g^c P + Kw^T V, E likewise with Y, mK, nk with the ones column
        // and y1; M += K^T Q undecayed
        const T *KA = DECAY ? sm.Kw : sm.K;
        const float gc = DECAY ? sm.gp[cv] : 1.f;
        for_blocks<PBk, NW>(w, [&](int pb, int ti0, int tv0) {
            if (DECAY) {
#pragma unroll
                for (int x = 0; x < PBk::BR * PBk::BR; ++x) {
                    (&accP[pb][0][0])[x] *= gc;
                    (&accE[pb][0][0])[x] *= gc;
                }
            }
            mma_tn_grp<PBk::BR, PBk::BR, C, TK, TV, false>(&accP[pb][0][0], KA, 16 * ti0, sm.V, 16 * tv0);
            mma_tn_grp<PBk::BR, PBk::BR, C, TK, TV, false>(&accE[pb][0][0], KA, 16 * ti0, sm.Y, 16 * tv0);
        });
        for_blocks<MBk, NW>(w, [&](int pb, int ti0, int tj0) {
            mma_tn_grp<MBk::BR, MBk::BR, C, TK, TK, false>(&accM[pb][0][0], sm.K, 16 * ti0, sm.Q, 16 * tj0);
        });
        for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
            if (DECAY) {
                accMK[j] *= gc;
                accNK[j] *= gc;
            }
            mma_tn_grp<1, 1, C, TK, TV, true>(&accMK[j], KA, 16 * ti, sm.V, 0);
            mma_tn_grp<1, 1, C, TK, TY1, false>(&accNK[j], KA, 16 * ti, sm.Y1, 0);
        });
        // the running widened P's T-typed copy after every product of the chunk
        for_owned<PBk, NW>(w, [&](int pb, int x, int y, int ti, int tv) {
            store4(sm.Pt + TK::off(16 * tv + col, 16 * ti + g4), accP[pb][x][y]);
        });
        for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
            store4(sm.Pt + TK::off(DV + col, 16 * ti + g4), accMK[j]);
        });
        c0 = n0;
        cv = ncv;
    }

    // summary [X = M | Y = P | N = E | y = mK | nv = nk]
    float *e = p.ws + node_offset(bh, 0, seg, p.BH, p.nreal, G::SUMF);
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
    for_stripe<G::UJ, NW, nTD>(w, [&](int j, int ti) {
        if (col == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[D * D + 2 * D * DV + 16 * ti + g4 + i] = accMK[j][i];
                e[D * D + 2 * D * DV + D + 16 * ti + g4 + i] = accNK[j][i];
            }
        }
    });
}

}  // namespace hla
