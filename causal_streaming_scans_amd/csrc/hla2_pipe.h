// hla2_pipe.h -- HLA-2 forward (stage 3) with the chunk loop software-pipelined
// by one chunk: between two barriers each wave forms the keyed queries Z of
// chunk j+1 and the read-out of chunk j, two independent chains of products.
//
// The operator and its streaming state are those of "1. HLA de Segundo Orden"
// ("Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
// gist.science/es/paper/2510.27258): with S = sum k k^T and W = sum z v^T
// (u = sum z), a chunk of tokens with carried (S0, W0, u0) gives
//     Z   = Q S0 + tril(Q K^T) K           (z_t = S_t q_t)
//     O   = Q W0 + tril(Q Z^T) V,  den = Q u0 + tril(Q Z^T) 1
//     S  <- S0 + K^T K,  W <- W0 + Z^T V,  u <- u0 + Z^T 1 .
// Z of chunk j+1 needs S after chunk j only, and the read-out of chunk j
// needs W before it, so the two can share a phase: per chunk there are two
// barriers instead of three, and every wave has two dependent chains to
// interleave.  The prefix fold and the state layout are the plain forward's.
//
// Buffers (LDS): K of chunk j+1; V and Z of chunks j and j+1 (double); the
// bf16 copies St = S after chunk j, Wt = W before chunk j (row DV: u).
//
// Iteration j (chunks j and j+1 both exist):
//   phase A  Z_{j+1} -> Z[(j+1)&1]; O_j (stored); W, u += Z_j^T [V_j | 1];
//            S += K_{j+1}^T K_{j+1}
//   barrier
//   phase B  St, Wt <- the new S, W, u; stage chunk j+2 (K, V[j&1], Q regs);
//            issue the loads of chunk j+3
//   barrier
// The output tile of each wave goes through LDS rows of its own, so the
// global stores write whole 128-byte rows; rows past the end of the sequence
// are dropped by the buffer resource's range check instead of a branch per
// tile, so each phase stays one basic block.
#pragma once

#include "hla2_kernels.h"

namespace hla {

template <typename T, int D, int DV, int C>
struct Hla2PipeSmem {
    using G = Hla2Cfg<T, D, DV, C, false>;
    alignas(16) T K[C * G::TK::LD];
    alignas(16) T V[2][C * G::TV::LD];
    alignas(16) T Z[2][C * G::TK::LD];
    alignas(16) T St[D * G::TS::LD];            // St[j][i] = S[i][j]
    alignas(16) T Wt[G::DVX * G::TS::LD];       // Wt[j][i] = W[i][j]; row DV = u
    alignas(16) T Ot[G::RT][16 * G::TV::LD];    // each wave's 16 output rows, on their way out
};

template <typename T, int D, int DV, int C>
using Hla2PipeLds = LdsWithScratch<Hla2PipeSmem<T, D, DV, C>, fold_scratch_floats<T, D, DV>()>;

// the shapes the pipelined loop is built for: bf16, one wave per row tile
template <typename T, int D, int DV, int C>
constexpr bool hla2_pipe_ok() {
    return sizeof(T) == 2 && Hla2Cfg<T, D, DV, C, false>::NCG == 1 &&
           sizeof(Hla2PipeLds<T, D, DV, C>) <= 80 * 1024;
}

// ZO: also write the keyed queries z_t = S_t q_t of every row to p.z_out.
template <typename T, int D, int DV, int C, bool ZO = false>
__global__ __launch_bounds__((Hla2Cfg<T, D, DV, C, false>::NT), 2)
void hla2_forward_pipe_kernel(FwdParams p) {
    using G = Hla2Cfg<T, D, DV, C, false>;
    constexpr int NT = G::NT, RT = G::RT, nTV = G::nTV;
    static_assert(G::NCG == 1, "one wave per row tile");
    using TK = typename G::TK;
    using TV = typename G::TV;
    using TS = typename G::TS;
    __shared__ Hla2PipeLds<T, D, DV, C> lds;
    auto &sm = lds.s;

    int seg, bh;
    forward_slot(p, blockIdx.x, &seg, &bh);
    const int w = wave_id();   // the wave's row tile
    const int col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.n, t_begin + p.seg_len);
    const int nch = (t_end - t_begin + C - 1) / C;
    const bool ratio = p.ratio != 0;
    const bool last = seg == p.nseg - 1;
    const T *q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    const T *k = static_cast<const T *>(p.k) + (size_t)bh * p.n * D;
    const T *v = static_cast<const T *>(p.v) + (size_t)bh * p.n * DV;
    T *o = static_cast<T *>(p.o) + (size_t)bh * p.n * DV;
    // this segment's rows of o; stores past its last valid row are dropped
    const __amdgpu_buffer_rsrc_t orsrc = rows_rsrc(o + (size_t)t_begin * DV, t_end - t_begin, DV);
    T *zo = ZO ? static_cast<T *>(p.z_out) + ((size_t)bh * p.n + t_begin) * D : nullptr;
    const __amdgpu_buffer_rsrc_t zrsrc = rows_rsrc(zo, ZO ? t_end - t_begin : 0, D);

    ChunkRegs<T, C, D, NT> rk;
    ChunkRegs<T, C, DV, NT> rv;
    RowFrags<T, D> qn;
    auto valid_of = [&](int c) { return min(C, t_end - (t_begin + C * c)); };
    auto load_chunk = [&](int c) {
        const int c0 = t_begin + C * c, valid = valid_of(c);
        const int tv = valid - 16 * w;
        qn.load_rows_g(q + (size_t)(c0 + (tv > 0 ? 16 * w : 0)) * D, D, tv > 0 ? tv : 0);
        rk.load(k + (size_t)c0 * D, valid);
        rv.load(v + (size_t)c0 * DV, valid);
    };

    const float *S0 = nullptr, *W0 = nullptr, *u0 = nullptr;
    if (p.state_in) {
        const float *e = p.state_in + (size_t)bh * G::STF;
        S0 = e;
        W0 = e + D * D;
        u0 = e + D * D + D * DV;
    }

    with_row_tile<RT>(w, [&](auto rt) {
        constexpr int R = decltype(rt)::value;
        using P = typename G::template FwdPlan<R>;
        const int tau = 16 * R + col;

        f32x4 acc[P::NA];
        for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = S0 ? S0[(16 * ti + g4 + i) * D + 16 * tj + col] : 0.f;
        });
        for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = W0 ? W0[(16 * ti + g4 + i) * DV + 16 * tv + col] : 0.f;
        });
        for_tiles<P, kU>(w, [&](int j, int ti, int) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = (u0 && col == 0) ? u0[16 * ti + g4 + i] : 0.f;
        });
        if (seg > 0) hla2_fold_prefix<T, D, DV, C, false, P>(p, bh, seg, 1.f, w, acc, lds.f);

        auto store_s = [&]() {
            for_tiles<P, kS>(w, [&](int j, int ti, int tj) {
                store4(sm.St + TS::off(16 * tj + col, 16 * ti + g4), acc[j]);
            });
        };
        auto store_w = [&]() {
            for_tiles<P, kW>(w, [&](int j, int ti, int tv) {
                store4(sm.Wt + TS::off(16 * tv + col, 16 * ti + g4), acc[j]);
            });
            for_tiles<P, kU>(w, [&](int j, int ti, int) {
                store4(sm.Wt + TS::off(DV + col, 16 * ti + g4), acc[j]);
            });
        };
        // S += K^T K over the staged chunk
        auto advance_s = [&]() {
            for_groups<P, kS, -1>(w, [&](auto gi, int ti0, int tj0) {
                constexpr Grp gr = P::grp(decltype(gi)::value);
                mma_tn_grp<gr.nr, gr.nc, C, TK, TK, false>(acc + gr.first, sm.K, 16 * ti0, sm.K, 16 * tj0);
            });
        };
        // W += Z^T V and u += Z^T 1 over chunk buffer b
        auto advance_w = [&](int b) {
            for_groups<P, kW, -1>(w, [&](auto gi, int ti0, int tj0) {
                constexpr Grp gr = P::grp(decltype(gi)::value);
                mma_tn_grp<gr.nr, gr.nc, C, TK, TV, false>(acc + gr.first, sm.Z[b], 16 * ti0, sm.V[b], 16 * tj0);
            });
            for_groups<P, kU, -1>(w, [&](auto gi, int ti0, int tj0) {
                constexpr Grp gr = P::grp(decltype(gi)::value);
                mma_tn_grp<gr.nr, gr.nc, C, TK, TV, true>(acc + gr.first, sm.Z[b], 16 * ti0, sm.V[b], 16 * tj0);
            });
        };
        // Z of the staged chunk c (queries qf) into Z[b]; with ZO this
        // wave's rows of it, which it wrote itself, also go out whole
        auto keyed = [&](const RowFrags<T, D> &qf, int b, int c) {
            Frag16<T> Lf[R + 1];
            scores_t<T, D, R, TK, false>(Lf, sm.K, qf, tau, nullptr, 1);
            z_tiles<T, D, R, 1, G::ZJ, TK, false, TS>(qf, Lf, sm.St, sm.K, sm.Z[b], nullptr, 1.f,
                                                      nullptr, 0, tau);
            if constexpr (ZO) store_rows_out<T, TK, D>(sm.Z[b] + 16 * R * TK::LD, zrsrc, C * c + 16 * R);
        };
        // o of chunk c (queries qf, keyed queries Z[b], values V[b]):
        // Q W0 + tril(Q Z^T) V, over Q u0 + tril(Q Z^T) 1 for the ratio form
        auto read_out = [&](const RowFrags<T, D> &qf, int b, int c) {
            f32x4 accO[nTV];
#pragma unroll
            for (int jv = 0; jv < nTV; ++jv) accO[jv] = mma_nt_ft<TS>(zero4(), sm.Wt + 16 * jv * TS::LD, qf);
            const f32x4 accD = mma_nt_ft<TS>(zero4(), sm.Wt + DV * TS::LD, qf);
            Frag16<T> Pf[R + 1];
            scores_t<T, D, R, TK, false>(Pf, sm.Z[b], qf, tau, nullptr, 2);
            f32x4 dc = zero4();
            const Frag16<T> ones = ones_frag<T>();
#pragma unroll
            for (int s = 0; s <= R; ++s) dc = mma16(dc, ones, Pf[s]);
            const float den = __shfl(accD[0] + dc[0], col);
            const float rden = ratio ? 1.f / den : 1.f;
            // the tile goes out through the wave's own LDS rows, whole rows at a time
            T *ot = sm.Ot[R];
#pragma unroll
            for (int jv = 0; jv < nTV; ++jv) {
                f32x4 oc = zero4();
#pragma unroll
                for (int s = 0; s <= R; ++s) oc = mma16(oc, ld_frag_tt<TV>(sm.V[b], 16 * s, 16 * jv), Pf[s]);
                store4(ot + TV::off(col, 16 * jv + g4), (accO[jv] + oc) * rden);
            }
            store_rows_out<T, TV, DV>(ot, orsrc, C * c + 16 * R);
        };

        store_s();
        store_w();
        RowFrags<T, D> qa, qb;   // Q of chunk j (read-out) and of chunk j+1 (keyed)
        if (nch > 0) {
            load_chunk(0);
            __syncthreads();   // copies written
            rk.template store_tile<TK>(sm.K);
            rv.template store_tile<TV>(sm.V[0]);
            qa = qn;
            qa.mask_rows(valid_of(0) - 16 * R);
            if (nch > 1) load_chunk(1);
            __syncthreads();
            keyed(qa, 0, 0);
            advance_s();
            __syncthreads();
            store_s();
            if (nch > 1) {
                rk.template store_tile<TK>(sm.K);
                rv.template store_tile<TV>(sm.V[1]);
                qb = qn;
                qb.mask_rows(valid_of(1) - 16 * R);
            }
            if (nch > 2) load_chunk(2);
            __syncthreads();
        }
        int j = 0;
        for (; j + 1 < nch; ++j) {
            const int b = j & 1;
            keyed(qb, b ^ 1, j + 1);
            read_out(qa, b, j);
            advance_w(b);
            advance_s();
            __syncthreads();
            store_s();
            store_w();
            qa = qb;
            if (j + 2 < nch) {
                rk.template store_tile<TK>(sm.K);
                rv.template store_tile<TV>(sm.V[b]);
                qb = qn;
                qb.mask_rows(valid_of(j + 2) - 16 * R);
            }
            if (j + 3 < nch) load_chunk(j + 3);
            __syncthreads();
        }
        if (nch > 0) read_out(qa, j & 1, j);

        if (p.state_out && last) {
            if (nch > 0) advance_w(j & 1);
            float *so = p.state_out + (size_t)bh * G::STF;
            for_tiles<P, kS>(w, [&](int jj, int ti, int tj) {
#pragma unroll
                for (int i = 0; i < 4; ++i) so[(16 * ti + g4 + i) * D + 16 * tj + col] = acc[jj][i];
            });
            for_tiles<P, kW>(w, [&](int jj, int ti, int tv) {
#pragma unroll
                for (int i = 0; i < 4; ++i) so[D * D + (16 * ti + g4 + i) * DV + 16 * tv + col] = acc[jj][i];
            });
            for_tiles<P, kU>(w, [&](int jj, int ti, int) {
                if (col == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) so[D * D + D * DV + 16 * ti + g4 + i] = acc[jj][i];
                }
            });
        }
    });
}

}  // namespace hla
