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
// a = g^(tokens in B) (1 without a decay):
//   HLA-2: X = a X_A + X_B, Y = a Y_A + Y_B, y = a y_A + y_B,
//          N = a^2 N_A + N_B + a X_A Y_B,  nv = a^2 nv_A + nv_B + a X_A y_B
//   AHLA : X = X_A + X_B (undecayed M), Y = a Y_A + Y_B, y = a y_A + y_B,
//          N = a N_A + N_B + a X_B Y_A,    nv = a nv_A + nv_B + a X_B y_A
//
// The scan's up-sweep runs over the stored summaries level by level, one
// launch per level and a few workgroups per combine (column slices): node
// (b, m) (layout in params.h) is the combine of its two children.  Its
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

// The right cross factor widened by one 16-column tile: [Y[:, c0 .. c0+CW) |
// y | 0 ...] into LDS [D][CW + 20], the vector column only when `with_vec`
// (else zeros).  One pass of 16-column tiles then gives the matrix and the
// vector cross terms together.
template <int D, int DV, int CW, int NT>
__device__ __forceinline__ void stage_right_ext(float *dst, const float *Y, int c0, const float *y,
                                                bool with_vec) {
    constexpr int LDB = CW + 20;
    static_assert(D <= NT, "one vector element per thread");
    // the vector element is loaded with the matrix, under the same wait
    const int t = threadIdx.x;
    float yv = 0.f;
    if (with_vec && t < D) yv = y[t];
    stage_f32<D, CW, NT>(dst, LDB, Y + c0, DV);
    // the rest of the widening tile is zero
    constexpr int NZ = D * 16, UZ = (NZ + NT - 1) / NT;
#pragma unroll
    for (int u = 0; u < UZ; ++u) {
        const int i = t + u * NT;
        if (i < NZ && (i % 16) != 0) dst[(i / 16) * LDB + CW + (i % 16)] = 0.f;
    }
    if (t < D) dst[t * LDB + CW] = yv;
}

// LDS floats of the staged factors: left [D][D + 4], right [D][CW + 20].
template <int D, int CW>
struct CrossLds {
    static constexpr int LDA = D + 4, LDB = CW + 20;
    static constexpr int FLOATS = D * LDA + D * LDB;
};

// A kernel's chunk buffers overlaid with the cross-factor staging area used
// before its first chunk.
template <typename S, int FLOATS>
union LdsWithScratch {
    S s;
    float f[FLOATS];
};

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

// Column slices a combine is split into (each a multiple of 16 columns).  At
// dv >= 128 a slice workgroup stages the whole d x d left factor (one per
// CU) and its products are fp32 MFMA chains over k = d, so eight slices of
// 1024 threads -- one tile per wave -- finish a level sooner than four of
// 256 (up-sweep of the d = 128 decay workload 39 -> 29 us).
template <int DV>
constexpr int combine_slices() { return DV / 16 < 4 ? DV / 16 : (DV >= 128 ? 8 : 4); }
template <int DV>
constexpr int combine_threads() { return DV >= 128 ? 1024 : 256; }

// Slice cs of eD = eA (+) eB, by all NT threads of the workgroup, eD a
// separate node (nothing is read that any slice writes).  The slice owns the
// columns [cs CW, (cs+1) CW) of Y and N, rows [cs D/CS, (cs+1) D/CS) of X,
// and (slice 0) y and nv.  `lds` holds CrossLds<D, CW>::FLOATS floats.  The
// staged factors and this wave's N / nv elements are loaded first; the linear
// parts are loaded once the staging has landed, under the MFMA work.
template <bool HLA2, int D, int DV, int NT, int CS>
__device__ void combine_slice(const float *eA, const float *eB, float *eD, float a, int cs,
                              float *lds) {
    using O = SumOfs<D, DV>;
    constexpr int CW = DV / CS;
    using L = CrossLds<D, CW>;
    constexpr int NW = NT / kWave, nTD = D / 16, nTW = CW / 16;
    constexpr int NTILE = nTD * (nTW + 1);   // N tiles of the slice, then the nv column
    constexpr int PT = (NTILE + NW - 1) / NW;
    const int w = wave_id(), col = acc_col(), g4 = (lane_id() >> 4) << 2;
    const int c0 = cs * CW;
    const bool first = cs == 0;
    const float *Xc = HLA2 ? eA + O::X : eB + O::X;
    const float *Yc = HLA2 ? eB + O::Y : eA + O::Y;
    const float *yc = HLA2 ? eB + O::y : eA + O::y;
    // scales of X, of Y and y, of N and nv, and of the cross term
    const float xs = HLA2 ? a : 1.f, ys = a, quad = HLA2 ? a * a : a, lin = a;
    float *As = lds, *Bs = lds + D * L::LDA;
    // which of this wave's tiles exist: the nv column only in slice 0
    auto tile_ok = [&](int t) { return t < nTD * nTW || (first && t < NTILE); };
    float na[PT][4], nb[PT][4];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = w + j * NW;
        if (tile_ok(t)) {
            const bool nvt = t >= nTD * nTW;
            const int ti = nvt ? t - nTD * nTW : t / nTW, tj = nvt ? 0 : t % nTW;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + g4 + i;
                const int idx = nvt ? O::nv + row : O::N + row * DV + c0 + 16 * tj + col;
                const bool use = !nvt || col == 0;
                na[j][i] = use ? eA[idx] : 0.f;
                nb[j][i] = use ? eB[idx] : 0.f;
            }
        }
    }
    stage_f32<D, D, NT>(As, L::LDA, Xc, D);
    stage_right_ext<D, DV, CW, NT>(Bs, Yc, c0, yc, first);
    __syncthreads();
    // linear parts of the slice: X rows [r0, r0 + D/CS), Y columns [c0, c0+CW), y
    constexpr int XR = D / CS, NX4 = XR * D / 4, NY4 = D * CW / 4;
    constexpr int UX = (NX4 + NT - 1) / NT, UY = (NY4 + NT - 1) / NT;
    const int r0 = cs * XR;
    f32x4 xa[UX], xb[UX], ya[UY], yb[UY];
#pragma unroll
    for (int u = 0; u < UX; ++u) {
        const int v = threadIdx.x + u * NT;
        if (v < NX4) {
            const int off = O::X + r0 * D + 4 * v;
            xa[u] = *reinterpret_cast<const f32x4 *>(eA + off);
            xb[u] = *reinterpret_cast<const f32x4 *>(eB + off);
        }
    }
#pragma unroll
    for (int u = 0; u < UY; ++u) {
        const int v = threadIdx.x + u * NT;
        if (v < NY4) {
            const int off = O::Y + (v / (CW / 4)) * DV + c0 + 4 * (v % (CW / 4));
            ya[u] = *reinterpret_cast<const f32x4 *>(eA + off);
            yb[u] = *reinterpret_cast<const f32x4 *>(eB + off);
        }
    }
    float vya = 0.f, vyb = 0.f;
    if (first && threadIdx.x < D) {
        vya = eA[O::y + threadIdx.x];
        vyb = eB[O::y + threadIdx.x];
    }
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = w + j * NW;
        if (tile_ok(t)) {
            const bool nvt = t >= nTD * nTW;
            const int ti = nvt ? t - nTD * nTW : t / nTW, tj = nvt ? nTW : t % nTW;
            const f32x4 cr = tile_ab_f32<D>(As + 16 * ti * L::LDA, L::LDA, Bs + 16 * tj, L::LDB);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + g4 + i;
                const float val = quad * na[j][i] + nb[j][i] + lin * cr[i];
                if (!nvt) eD[O::N + row * DV + c0 + 16 * tj + col] = val;
                else if (col == 0) eD[O::nv + row] = val;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < UX; ++u) {
        const int v = threadIdx.x + u * NT;
        if (v < NX4) *reinterpret_cast<f32x4 *>(eD + O::X + r0 * D + 4 * v) = xs * xa[u] + xb[u];
    }
#pragma unroll
    for (int u = 0; u < UY; ++u) {
        const int v = threadIdx.x + u * NT;
        if (v < NY4) {
            const int off = O::Y + (v / (CW / 4)) * DV + c0 + 4 * (v % (CW / 4));
            *reinterpret_cast<f32x4 *>(eD + off) = ys * ya[u] + yb[u];
        }
    }
    if (first && threadIdx.x < D) eD[O::y + threadIdx.x] = ys * vya + vyb;
}

// Workgroups of one up-sweep level: the CS column slices of a combine are
// 8 workgroup ids apart, so they run on one XCD (ids are dealt to the XCDs
// in turn) and the left factor they all read is fetched into its L2 once.
// Combine c = bh * npair + m; ids past the last combine exit at once.
template <int CS>
__host__ __device__ inline int up_sweep_groups(int ncomb) { return ((ncomb + 7) / 8) * 8 * CS; }
template <int CS>
__device__ inline void up_sweep_slot(int id, int *comb, int *cs) {
    *comb = (id / (8 * CS)) * 8 + id % 8;
    *cs = (id / 8) % CS;
}

// One level of the up-sweep of the exclusive Blelloch scan: a workgroup forms
// column slice cs of node (b+1, m) of head bh from its children (b, 2m) and
// (b, 2m+1).  The host launches the levels in order, one launch each, over
// the nodes that end below nreal (a node ending at or past it would only feed
// prefixes no segment needs).
template <bool HLA2, int D, int DV, int NT>
__global__ __launch_bounds__(NT) void up_sweep_kernel(FwdParams p, int b) {
    constexpr int SUMF = summary_floats(D, DV);
    constexpr int CS = combine_slices<DV>();
    __shared__ alignas(16) float lds[CrossLds<D, DV / CS>::FLOATS];
    const int npair = p.nreal >> (b + 1);
    int comb, cs;
    up_sweep_slot<CS>(blockIdx.x, &comb, &cs);
    if (comb >= npair * p.BH) return;
    const int bh = comb / npair, m = comb - bh * npair;
    // every entry is 1 without a decay, so a is exactly 1 then
    const float g = p.gamma[gamma_slot(bh, p.H)];
    const float a = pow_int(g, (long)p.seg_len << b);   // g^(tokens of a child)
    combine_slice<HLA2, D, DV, NT, CS>(p.ws + node_offset(bh, b, 2 * m, p.BH, p.nreal, SUMF),
                                       p.ws + node_offset(bh, b, 2 * m + 1, p.BH, p.nreal, SUMF),
                                       p.ws + node_offset(bh, b + 1, m, p.BH, p.nreal, SUMF), a, cs,
                                       lds);
}

}  // namespace hla
