// unmasked.hip -- the unmasked (non-causal) second-order operators, and their
// C entry points (declared in include/hla.h).
//
// Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
// (gist.science/es/paper/2510.27258).  Without the causal masks the
// second-order operator of "1. HLA de Segundo Orden" is the product of the
// prefix moments taken over the whole sequence, and the asymmetric operator
// of "2. ... (AHLA)" likewise:
//     HLA-2:  o = (Q K^T)(K Q^T) V = Q (K^T K)(Q^T V)
//     AHLA :  o = (Q K^T)(Q K^T) V = Q (K^T Q)(K^T V)
// Both are o_t = T^T q_t with one d x d matrix T = G1 G2 per head, where G1,
// G2 are token sums of outer products (G1 = X^T Y, G2 = U^T W).  Three
// launches: per-block partial sums of G1 and G2, their fixed-order sum and
// product T, and the per-row read-out.  fp32 arithmetic, except that for
// bf16 inputs the moment sums and (d >= 32) the read-out run on bf16 MFMA
// with fp32 accumulation, the read-out with T rounded to bf16.
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/hla.h"
#include "device_common.h"

namespace hla {
namespace {

struct UnmaskedParams {
    const void *x, *y, *u, *w;   // [BH][n][D] operands of G1 = X^T Y, G2 = U^T W
    const void *q;               // [BH][n][D] queries of the read-out
    void *o;                     // [BH][n][D] output
    float *partial;              // [BH][nblk][2][D][D]
    float *tmat;                 // [BH][D][D]
    bf16 *tmat_t;                // [BH][D][D] T transposed, bf16 (MFMA read-out)
    long n;
    int BH, nblk;
};

constexpr int kUnmaskedMaxBlocks = 64;   // partial-sum workgroups per head, at most

// Workgroups per head of the partial-sum launch: about 512 in all, each over
// at least 32 tokens.
long unmasked_blocks(long BH, long n) {
    long nb = (512 + BH - 1) / BH;
    const long by_len = (n + 31) / 32;
    if (nb > by_len) nb = by_len;
    if (nb > kUnmaskedMaxBlocks) nb = kUnmaskedMaxBlocks;
    return nb < 1 ? 1 : nb;
}

template <typename T> __device__ __forceinline__ f32x4 ld4(const T *p);
template <> __device__ __forceinline__ f32x4 ld4<bf16>(const bf16 *p) {
    union { uint2 u; bf16 h[4]; } x;
    x.u = *reinterpret_cast<const uint2 *>(p);
    return f32x4{(float)x.h[0], (float)x.h[1], (float)x.h[2], (float)x.h[3]};
}
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}

// Step 1: workgroup (x, bh) sums x_t y_t^T and u_t w_t^T over its token range
// (32-token tiles staged in LDS as fp32).  Thread i owns the 4 x 4 blocks
// i, i + 256, ... of both matrices.
template <typename T, int D>
__global__ __launch_bounds__(256) void unmasked_gram_kernel(UnmaskedParams p) {
    constexpr int TT = 32, NBD = D / 4, NB = NBD * NBD, BPT = (NB + 255) / 256;
    __shared__ alignas(16) float sx[TT][D], sy[TT][D], su[TT][D], sw[TT][D];
    const int bh = blockIdx.y, tid = threadIdx.x;
    const long per = (p.n + p.nblk - 1) / p.nblk;
    const long t_begin = (long)blockIdx.x * per;
    const long t_end = min(p.n, t_begin + per);
    const size_t head = (size_t)bh * p.n * D;
    const T *X = static_cast<const T *>(p.x) + head, *Y = static_cast<const T *>(p.y) + head;
    const T *U = static_cast<const T *>(p.u) + head, *W = static_cast<const T *>(p.w) + head;
    float a1[BPT][4][4], a2[BPT][4][4];
#pragma unroll
    for (int m = 0; m < BPT; ++m)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) a1[m][a][b] = a2[m][a][b] = 0.f;
    for (long t0 = t_begin; t0 < t_end; t0 += TT) {
        for (int e = tid; e < TT * NBD; e += 256) {
            const int r = e / NBD, c = 4 * (e % NBD);
            const long t = t0 + r;
            const bool ok = t < t_end;
            const size_t off = (size_t)t * D + c;
            *reinterpret_cast<f32x4 *>(&sx[r][c]) = ok ? ld4(X + off) : f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4 *>(&sy[r][c]) = ok ? ld4(Y + off) : f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4 *>(&su[r][c]) = ok ? ld4(U + off) : f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4 *>(&sw[r][c]) = ok ? ld4(W + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        for (int r = 0; r < TT; ++r) {
#pragma unroll
            for (int m = 0; m < BPT; ++m) {
                const int bidx = tid + 256 * m;
                if (bidx < NB) {
                    const int bi = 4 * (bidx / NBD), bj = 4 * (bidx % NBD);
                    const f32x4 xv = *reinterpret_cast<const f32x4 *>(&sx[r][bi]);
                    const f32x4 yv = *reinterpret_cast<const f32x4 *>(&sy[r][bj]);
                    const f32x4 uv = *reinterpret_cast<const f32x4 *>(&su[r][bi]);
                    const f32x4 wv = *reinterpret_cast<const f32x4 *>(&sw[r][bj]);
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            a1[m][a][b] += xv[a] * yv[b];
                            a2[m][a][b] += uv[a] * wv[b];
                        }
                }
            }
        }
        __syncthreads();
    }
    float *out = p.partial + ((size_t)bh * p.nblk + blockIdx.x) * 2 * D * D;
#pragma unroll
    for (int m = 0; m < BPT; ++m) {
        const int bidx = tid + 256 * m;
        if (bidx < NB) {
            const int bi = 4 * (bidx / NBD), bj = 4 * (bidx % NBD);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                *reinterpret_cast<f32x4 *>(out + (bi + a) * D + bj) =
                    f32x4{a1[m][a][0], a1[m][a][1], a1[m][a][2], a1[m][a][3]};
                *reinterpret_cast<f32x4 *>(out + D * D + (bi + a) * D + bj) =
                    f32x4{a2[m][a][0], a2[m][a][1], a2[m][a][2], a2[m][a][3]};
            }
        }
    }
}

// Step 1 for bf16 inputs, on the matrix cores: the same sums as
// unmasked_gram_kernel, G[i][j] += sum_t x_t[i] y_t[j], as 16 x 16 tiles of
// mfma_f32_16x16x32_bf16 over 64-token tiles.  Each tile is staged
// row-major ([token][feature], LdsTile layout) with 16-byte copies, and both
// operands (8 consecutive tokens of one feature per lane) come from the
// transposing LDS read.  The next tile's rows are loaded into registers
// while the current one is multiplied, and an operand that is another one's
// tensor (K in K^T K; K in both moments of AHLA) is loaded and staged once.
// Wave w owns tiles w, w + 4, ... of [G1 tiles | G2 tiles]; accumulator
// element r of lane l is G[16 ti + 4 (l / 16) + r][16 tj + l % 16].
template <int D>
__global__ __launch_bounds__(256) void unmasked_gram_mfma_kernel(UnmaskedParams p) {
    using TL = LdsTile<bf16, D>;
    constexpr int TT = 64, NTD = D / 16, NT1 = NTD * NTD, NT = 2 * NT1;
    constexpr int TPW = (NT + 3) / 4;
    constexpr int VPR = D / 8, NVEC = TT * VPR, NV = (NVEC + 255) / 256;   // 16-byte pieces
    __shared__ alignas(16) bf16 tiles[4][TT * TL::LD];
    const int bh = blockIdx.y, tid = threadIdx.x, l = lane_id(), w = wave_id();
    const long per = (p.n + p.nblk - 1) / p.nblk;
    const long t_begin = (long)blockIdx.x * per;
    const long t_end = min(p.n, t_begin + per);
    const size_t head = (size_t)bh * p.n * D;
    const bf16 *src[4] = {static_cast<const bf16 *>(p.x) + head, static_cast<const bf16 *>(p.y) + head,
                          static_cast<const bf16 *>(p.u) + head, static_cast<const bf16 *>(p.w) + head};
    // LDS tile of each operand: a tensor that equals an earlier operand's
    // shares its tile (wave-uniform: kernel arguments only)
    const int slot[4] = {0, p.y == p.x ? 0 : 1, p.u == p.x ? 0 : (p.u == p.y ? 1 : 2),
                         p.w == p.x ? 0 : (p.w == p.y ? 1 : (p.w == p.u ? 2 : 3))};
    uint4 rg[4][NV];
    auto load = [&](long t0) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if (slot[a] != a) continue;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = tid + 256 * i, r = e / VPR, c = 8 * (e % VPR);
                const long t = t0 + r;
                // a row past the range reads the range's first row (in bounds)
                // and is stored as zeros
                const long tr = (e < NVEC && t < t_end) ? t : t_begin;
                rg[a][i] = *reinterpret_cast<const uint4 *>(src[a] + (size_t)tr * D + (e < NVEC ? c : 0));
            }
        }
    };
    auto stage = [&](long t0) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if (slot[a] != a) continue;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = tid + 256 * i, r = e / VPR, c = 8 * (e % VPR);
                if (e < NVEC) {
                    const unsigned m = t0 + r < t_end ? 0xffffffffu : 0u;
                    uint4 x = rg[a][i];
                    x.x &= m; x.y &= m; x.z &= m; x.w &= m;
                    *reinterpret_cast<uint4 *>(&tiles[a][TL::off(r, c)]) = x;
                }
            }
        }
    };
    f32x4 acc[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t_begin < t_end) load(t_begin);
    for (long t0 = t_begin; t0 < t_end; t0 += TT) {
        __syncthreads();   // the previous tile's readers are done
        stage(t0);
        if (t0 + TT < t_end) load(t0 + TT);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int tau = w + 4 * m;
            if (tau < NT) {
                const int mat = tau / NT1, rem = tau % NT1;
                const int ti = rem / NTD, tj = rem % NTD;
                const bf16 *A = tiles[slot[mat == 0 ? 0 : 2]], *Bm = tiles[slot[mat == 0 ? 1 : 3]];
#pragma unroll
                for (int k0 = 0; k0 < TT; k0 += 32)
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_op8_tt<TL>(A, k0, 16 * ti),
                                                                     ld_op8_tt<TL>(Bm, k0, 16 * tj), acc[m], 0, 0, 0);
            }
        }
    }
    float *out = p.partial + ((size_t)bh * p.nblk + blockIdx.x) * 2 * D * D;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int tau = w + 4 * m;
        if (tau < NT) {
            const int mat = tau / NT1, rem = tau % NT1;
            const int ti = rem / NTD, tj = rem % NTD;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[mat * D * D + (16 * ti + 4 * (l >> 4) + r) * D + 16 * tj + (l & 15)] = acc[m][r];
        }
    }
}

// Step 2: workgroup bh sums its partials in block order and forms T = G1 G2.
// The sums run over 16-byte pieces with every block's loads in flight
// together; G1 is kept transposed so that each thread's 4 x 4 block of T
// reads one 16-byte piece of each factor per step over m.
template <int D>
__global__ __launch_bounds__(256) void unmasked_product_kernel(UnmaskedParams p) {
    constexpr int Q4 = D * D / 4, NBK = (D / 4) * (D / 4), BPT = (NBK + 255) / 256;
    __shared__ alignas(16) float g1t[D * D], g2[D * D];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const float *part = p.partial + (size_t)bh * p.nblk * 2 * D * D;
    for (int e = tid; e < Q4; e += 256) {
        f32x4 s1 = zero4(), s2 = zero4();
        int x = 0;
        for (; x + 4 <= p.nblk; x += 4) {
            f32x4 a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = *reinterpret_cast<const f32x4 *>(part + (size_t)(x + u) * 2 * D * D + 4 * e);
                b[u] = *reinterpret_cast<const f32x4 *>(part + (size_t)(x + u) * 2 * D * D + D * D + 4 * e);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                s1 += a[u];
                s2 += b[u];
            }
        }
        for (; x < p.nblk; ++x) {
            s1 += *reinterpret_cast<const f32x4 *>(part + (size_t)x * 2 * D * D + 4 * e);
            s2 += *reinterpret_cast<const f32x4 *>(part + (size_t)x * 2 * D * D + D * D + 4 * e);
        }
        const int i = (4 * e) / D, j = (4 * e) % D;
#pragma unroll
        for (int c = 0; c < 4; ++c) g1t[(j + c) * D + i] = s1[c];
        *reinterpret_cast<f32x4 *>(&g2[4 * e]) = s2;
    }
    __syncthreads();
    float *Tm = p.tmat + (size_t)bh * D * D;
    bf16 *Tt = p.tmat_t + (size_t)bh * D * D;
#pragma unroll
    for (int bb = 0; bb < BPT; ++bb) {
        const int blk = tid + 256 * bb;
        if (blk < NBK) {
            const int i0 = 4 * (blk / (D / 4)), j0 = 4 * (blk % (D / 4));
            f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
            for (int m = 0; m < D; ++m) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&g1t[m * D + i0]);
                const f32x4 b = *reinterpret_cast<const f32x4 *>(&g2[m * D + j0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += a[r] * b;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) *reinterpret_cast<f32x4 *>(Tm + (i0 + r) * D + j0) = acc[r];
            // T^T rows j0 .. j0+3, columns i0 .. i0+3, in bf16
#pragma unroll
            for (int c = 0; c < 4; ++c)
                store4(Tt + (j0 + c) * D + i0, f32x4{acc[0][c], acc[1][c], acc[2][c], acc[3][c]});
        }
    }
}

// Step 3 for bf16 inputs and D >= 32, on the matrix cores: o = Q T with T
// rounded to bf16.  Wave w forms tokens t0 + 16 w .. + 15, all D columns, as
// D/16 tiles of o^T = T^T Q^T on mfma_f32_16x16x32_bf16: lane l's operands
// are 8 consecutive rows of column 16 tj + l % 16 of T, i.e. a 16-byte piece
// of a row of T^T (staged in LDS), and 8 consecutive features of token
// 16 w + l % 16 (one 16-byte load from HBM); accumulator r is column
// 16 tj + 4 (l / 16) + r of that token.  The wave's 16 rows of o go through
// LDS rows of its own and out as whole rows (stores past the sequence are
// dropped by the buffer resource's range check).
template <int D>
__global__ __launch_bounds__(256) void unmasked_apply_mfma_kernel(UnmaskedParams p) {
    constexpr int NTD = D / 16, LD = D + 8;
    using TO = LdsTile<bf16, D>;
    __shared__ alignas(16) bf16 tt[D][LD];
    __shared__ alignas(16) bf16 ost[4][16 * TO::LD];
    const int bh = blockIdx.y, tid = threadIdx.x, l = lane_id(), w = wave_id();
    const bf16 *Tt = p.tmat_t + (size_t)bh * D * D;
    for (int e = tid; e < D * D / 8; e += 256) {
        const int r = e / (D / 8), c = 8 * (e % (D / 8));
        *reinterpret_cast<bf16x8 *>(&tt[r][c]) = *reinterpret_cast<const bf16x8 *>(Tt + r * D + c);
    }
    __syncthreads();
    const long t0 = (long)blockIdx.x * 64 + 16 * w;
    const long ta = t0 + (l & 15);
    const bf16 *Q = static_cast<const bf16 *>(p.q) + (size_t)bh * p.n * D;
    f32x4 acc[NTD];
#pragma unroll
    for (int j = 0; j < NTD; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D; ks += 32) {
        const bf16x8 a = ta < p.n ? *reinterpret_cast<const bf16x8 *>(Q + (size_t)ta * D + ks + 8 * (l >> 4))
                                  : bf16x8{};
#pragma unroll
        for (int j = 0; j < NTD; ++j) {
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(&tt[16 * j + (l & 15)][ks + 8 * (l >> 4)]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, acc[j], 0, 0, 0);
        }
    }
    bf16 *O = static_cast<bf16 *>(p.o) + (size_t)bh * p.n * D;
    bf16 *ot = ost[w];
#pragma unroll
    for (int j = 0; j < NTD; ++j) store4(ot + TO::off(l & 15, 16 * j + 4 * (l >> 4)), acc[j]);
    const long valid = p.n - t0;
    const __amdgpu_buffer_rsrc_t rs =
        rows_rsrc(O + (size_t)t0 * D, valid <= 0 ? 0 : (valid < 16 ? (int)valid : 16), D);
    store_rows_out<bf16, TO, D>(ot, rs, 0);
}

// Step 3: workgroup (x, bh) writes o_t = T^T q_t for 64 tokens; thread
// (r, c) forms columns c*D/4 .. of token r.
template <typename T, int D>
__global__ __launch_bounds__(256) void unmasked_apply_kernel(UnmaskedParams p) {
    constexpr int QC = D / 4;
    __shared__ alignas(16) float tm[D * D];
    __shared__ float sq[64][D + 1];
    const int bh = blockIdx.y, tid = threadIdx.x;
    const long t0 = (long)blockIdx.x * 64;
    const float *Tm = p.tmat + (size_t)bh * D * D;
    for (int e = tid; e < D * D / 4; e += 256)
        *reinterpret_cast<f32x4 *>(&tm[4 * e]) = *reinterpret_cast<const f32x4 *>(Tm + 4 * e);
    const T *Q = static_cast<const T *>(p.q) + (size_t)bh * p.n * D;
    for (int e = tid; e < 64 * (D / 4); e += 256) {
        const int r = e / (D / 4), c = 4 * (e % (D / 4));
        const long t = t0 + r;
        const f32x4 v = t < p.n ? ld4(Q + (size_t)t * D + c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) sq[r][c + j] = v[j];
    }
    __syncthreads();
    const int r = tid / 4, c = tid % 4;
    float acc[QC];
#pragma unroll
    for (int j = 0; j < QC; ++j) acc[j] = 0.f;
    for (int i = 0; i < D; ++i) {
        const float qi = sq[r][i];
#pragma unroll
        for (int j = 0; j < QC; ++j) acc[j] += qi * tm[i * D + c * QC + j];
    }
    const long t = t0 + r;
    if (t < p.n) {
        T *O = static_cast<T *>(p.o) + ((size_t)bh * p.n + t) * D + c * QC;
#pragma unroll
        for (int j = 0; j < QC; ++j) O[j] = from_f<T>(acc[j]);
    }
}

template <typename T, int D>
hipError_t launch_unmasked(const UnmaskedParams &p, hipStream_t s) {
    if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((unmasked_gram_mfma_kernel<D>), dim3((unsigned)p.nblk, (unsigned)p.BH),
                           dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((unmasked_gram_kernel<T, D>), dim3((unsigned)p.nblk, (unsigned)p.BH),
                           dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((unmasked_product_kernel<D>), dim3((unsigned)p.BH), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((p.n + 63) / 64), (unsigned)p.BH);
    if constexpr (sizeof(T) == 2 && D >= 32)
        hipLaunchKernelGGL((unmasked_apply_mfma_kernel<D>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((unmasked_apply_kernel<T, D>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

typedef hipError_t (*UnmaskedLaunch)(const UnmaskedParams &, hipStream_t);

UnmaskedLaunch lookup_unmasked(int dtype, int d) {
    if (dtype == HLA_F32) {
        switch (d) {
            case 16: return launch_unmasked<float, 16>;
            case 32: return launch_unmasked<float, 32>;
            case 64: return launch_unmasked<float, 64>;
            case 128: return launch_unmasked<float, 128>;
        }
        return nullptr;
    }
    switch (d) {
        case 16: return launch_unmasked<bf16, 16>;
        case 32: return launch_unmasked<bf16, 32>;
        case 64: return launch_unmasked<bf16, 64>;
        case 128: return launch_unmasked<bf16, 128>;
    }
    return nullptr;
}

}  // namespace
}  // namespace hla

using namespace hla;

extern "C" {

size_t hla_unmasked_workspace_bytes(int B, int H, int n, int d) {
    if (B < 1 || H < 1 || n < 1 || d < 1) return 0;
    const long BH = (long)B * H;
    const long nb = unmasked_blocks(BH, n);
    return (size_t)BH * (size_t)(2 * nb + 1) * d * d * sizeof(float) +
           (size_t)BH * d * d * sizeof(bf16);
}

hla_status hla_unmasked_forward(const void *q, const void *k, const void *v, void *o, int B,
                                int H, int n, int d, int dtype, int variant, void *workspace,
                                size_t workspace_bytes, void *stream) {
    if (dtype != HLA_F32 && dtype != HLA_BF16) return HLA_ERR_ARG;
    if (variant < HLA_HLA2 || variant > HLA_HLA3) return HLA_ERR_ARG;
    if (B < 1 || H < 1 || d < 1 || n < 0) return HLA_ERR_SHAPE;
    if (variant != HLA_HLA2 && variant != HLA_AHLA) return HLA_ERR_UNSUPPORTED;
    if ((long)B * H > 65535) return HLA_ERR_UNSUPPORTED;
    const UnmaskedLaunch fn = lookup_unmasked(dtype, d);
    if (!fn) return HLA_ERR_UNSUPPORTED;
    if ((n + 63L) / 64 > INT32_MAX / 2) return HLA_ERR_UNSUPPORTED;
    if (n == 0) return HLA_OK;
    if (!q || !k || !v || !o) return HLA_ERR_NULL;
    if (!workspace) return HLA_ERR_NULL;
    if (workspace_bytes < hla_unmasked_workspace_bytes(B, H, n, d)) return HLA_ERR_WORKSPACE;
    UnmaskedParams p;
    memset(&p, 0, sizeof(p));
    const bool hla2 = variant == HLA_HLA2;
    p.x = k;                      // G1 = K^T K (HLA-2) or K^T Q (AHLA)
    p.y = hla2 ? k : q;
    p.u = hla2 ? q : k;           // G2 = Q^T V (HLA-2) or K^T V (AHLA)
    p.w = v;
    p.q = q;
    p.o = o;
    p.BH = B * H;
    p.n = n;
    p.nblk = (int)unmasked_blocks(p.BH, n);
    p.partial = static_cast<float *>(workspace);
    p.tmat = p.partial + (size_t)p.BH * p.nblk * 2 * d * d;
    p.tmat_t = reinterpret_cast<bf16 *>(p.tmat + (size_t)p.BH * d * d);
    return fn(p, static_cast<hipStream_t>(stream)) == hipSuccess ? HLA_OK : HLA_ERR_DEVICE;
}

}  // extern "C"
