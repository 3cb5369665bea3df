// combine.h -- the semidirect-product combine of segment summaries and the
// up-sweep of the exclusive Blelloch scan (gfx950).
//
// Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
// gist.science/es/paper/2510.27258, section "4. Entrenamiento Paralelo
// mediante Escaneos Asociativos": segments are concatenated by an associative
// semidirect-product operator whose cross terms pair one segment's key moment
// with the other's query-value moment, and an exclusive Blelloch scan over
// the segment summaries reproduces the serial recurrence exactly.
//
// Summary = (X, Y, N, y, nv) (layout in params.h).  Combine, A earlier than B,
// a = g^(tokens in B) (1 for AHLA):
//   HLA-2: X = a X_A + X_B, Y = a Y_A + Y_B, y = a y_A + y_B,
//          N = a^2 N_A + N_B + a X_A Y_B,  nv = a^2 nv_A + nv_B + a X_A y_B
//   AHLA : X = X_A + X_B, Y = Y_A + Y_B, y = y_A + y_B,
//          N = N_A + N_B + X_B Y_A,        nv = nv_A + nv_B + X_B y_A
//
// The scan's up-sweep runs as its own kernel over the stored summaries, one
// workgroup per (b,h), level by level: node (b, m) (layout in params.h) is
// the combine of its two children, written over the right child.  Its
// down-sweep is never materialised: the exclusive prefix of segment s is the
// combine, left to right, of the up-sweep nodes that tile [0, s) -- one per
// set bit of s, largest first -- and each forward workgroup forms its own
// from the stored nodes, folding them into its carried state before its
// first chunk.  That is the value the down-sweep would deliver to leaf s.
//
// Cross terms run on V_MFMA_F32_16X16X4_F32: exact fp32 products, fp32 sums.
#pragma once

#include "device_common.h"
#include "params.h"

namespace hla {

// LDS staging of the two cross-term factors, fp32: the left factor as
// [D][D + 4] and the right factor widened to [D][DV + 20] -- its DV columns,
// then the vector (y or mK) as column DV, then 15 zero columns -- so one
// pass of 16-column tiles gives both the matrix and the vector cross terms.
template <int D, int DV>
struct CrossLds {
    static constexpr int LDA = D + 4, LDB = DV + 20;
    static constexpr int FLOATS = D * LDA + D * LDB;
};

// A kernel's chunk buffers overlaid with the cross-factor staging area used
// before its first chunk.
template <typename S, int FLOATS>
union LdsWithScratch {
    S s;
    float f[FLOATS];
};

// dst[r][c] = src[r][c] for a [ROWS][COLS] fp32 block (COLS a multiple of 4),
// float4-wise by NT threads, every load issued before any store.
template <int ROWS, int COLS, int NT>
__device__ __forceinline__ void stage_f32(float *dst, int ldd, const float *src, int lds) {
    constexpr int V4 = COLS / 4, NV = ROWS * V4, U = (NV + NT - 1) / NT;
    f32x4 buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int idx = threadIdx.x + u * NT;
        if (idx < NV) buf[u] = *reinterpret_cast<const f32x4 *>(src + (size_t)(idx / V4) * lds + 4 * (idx % V4));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int idx = threadIdx.x + u * NT;
        if (idx < NV) *reinterpret_cast<f32x4 *>(dst + (idx / V4) * ldd + 4 * (idx % V4)) = buf[u];
    }
}

// the widened right factor [Y | y | 0 ...] of a summary into LDS
template <int D, int DV, int NT>
__device__ __forceinline__ void stage_right_ext(float *dst, const float *Y, const float *y) {
    constexpr int LDB = CrossLds<D, DV>::LDB;
    stage_f32<D, DV, NT>(dst, LDB, Y, DV);
    for (int i = threadIdx.x; i < D * 16; i += NT)
        dst[(i / 16) * LDB + DV + (i % 16)] = (i % 16) == 0 ? y[i / 16] : 0.f;
}

// 16x16 tile of A B, A [16 rows][K] row-major (lda, rows 16-byte aligned),
// B [K][16 columns] row-major (ldb), both in LDS.  Lane (c, g) pairs
// A[c][k0 + 4g + m] with B[k0 + 4g + m][c] in instruction m, so both sides
// see the same k.
template <int K>
__device__ __forceinline__ f32x4 tile_ab_f32(const float *A, int lda, const float *B, int ldb) {
    const int l = lane_id(), c = l & 15, g = l >> 4;
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(A + c * lda + k0 + 4 * g);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], B[(k0 + 4 * g + m) * ldb + c], acc, 0, 0, 0);
    }
    return acc;
}

// eB <- eA (+) eB for two summaries in global memory, in place, by all NT
// threads of the workgroup; `lds` holds CrossLds<D, DV>::FLOATS floats.
// The cross factors are staged first, so every later global access of a
// thread touches only the elements that thread itself rewrites.
template <bool HLA2, int D, int DV, int NT>
__device__ void combine_nodes(const float *eA, float *eB, float a, float *lds) {
    using O = SumOfs<D, DV>;
    using L = CrossLds<D, DV>;
    constexpr int NW = NT / kWave, nTD = D / 16, nTV = DV / 16;
    constexpr int NTILE = nTD * (nTV + 1);   // N tiles, then the nv column per row tile
    constexpr int PT = (NTILE + NW - 1) / NW;
    const int w = wave_id(), col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const float *Xc = HLA2 ? eA + O::X : eB + O::X;
    const float *Yc = HLA2 ? eB + O::Y : eA + O::Y;
    const float *yc = HLA2 ? eB + O::y : eA + O::y;
    const float lin = HLA2 ? a : 1.f, quad = HLA2 ? a * a : 1.f;
    float *As = lds, *Bs = lds + D * L::LDA;
    stage_f32<D, D, NT>(As, L::LDA, Xc, D);
    stage_right_ext<D, DV, NT>(Bs, Yc, yc);
    // this wave's N / nv elements of both operands, loaded while staging lands
    float na[PT][4], nb[PT][4];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = w + j * NW;
        if (t < NTILE) {
            const int ti = t / (nTV + 1), tj = t % (nTV + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + g4 + i;
                const int idx = tj < nTV ? O::N + row * DV + 16 * tj + col : O::nv + row;
                const bool use = tj < nTV || col == 0;
                na[j][i] = use ? eA[idx] : 0.f;
                nb[j][i] = use ? eB[idx] : 0.f;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = w + j * NW;
        if (t < NTILE) {
            const int ti = t / (nTV + 1), tj = t % (nTV + 1);
            const f32x4 cr = tile_ab_f32<D>(As + 16 * ti * L::LDA, L::LDA, Bs + 16 * tj, L::LDB);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + g4 + i;
                const float val = quad * na[j][i] + nb[j][i] + lin * cr[i];
                if (tj < nTV) eB[O::N + row * DV + 16 * tj + col] = val;
                else if (col == 0) eB[O::nv + row] = val;
            }
        }
    }
    // X and Y are adjacent: one float4 pass, then y
    constexpr int NXY4 = (D * D + D * DV) / 4;
    const f32x4 *A4 = reinterpret_cast<const f32x4 *>(eA);
    f32x4 *B4 = reinterpret_cast<f32x4 *>(eB);
    for (int v = threadIdx.x; v < NXY4; v += NT) B4[v] = lin * A4[v] + B4[v];
    for (int i = threadIdx.x; i < D; i += NT) eB[O::y + i] = lin * eA[O::y + i] + eB[O::y + i];
}

// Up-sweep of the exclusive Blelloch scan for head blockIdx.x: every node
// whose segments all have summaries, lowest level first.  A node that ends
// at or past nreal would only feed prefixes no segment needs.
template <bool HLA2, int D, int DV, int NT>
__global__ __launch_bounds__(NT) void up_sweep_kernel(FwdParams p) {
    constexpr int SUMF = summary_floats(D, DV);
    __shared__ alignas(16) float lds[CrossLds<D, DV>::FLOATS];
    const int bh = blockIdx.x;
    float *base = p.ws + ws_node(bh, 0, p.nreal, SUMF);
    const float g = HLA2 ? p.gamma[bh % p.H] : 1.f;
    for (int b = 0; node_slot(b + 1, 0) <= p.nreal - 1; ++b) {
        const float a = HLA2 ? pow_int(g, (long)p.seg_len << b) : 1.f;   // g^(tokens of a child)
        for (int m = 0; node_slot(b + 1, m) <= p.nreal - 1; ++m) {
            combine_nodes<HLA2, D, DV, NT>(base + (size_t)node_slot(b, 2 * m) * SUMF,
                                           base + (size_t)node_slot(b, 2 * m + 1) * SUMF, a, lds);
            __syncthreads();   // the parent is complete before anything reads it
        }
    }
}

}  // namespace hla
