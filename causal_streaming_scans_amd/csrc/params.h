// params.h -- kernel argument block and workspace layout (internal).
#pragma once

#include <stddef.h>

namespace hla {

constexpr int kMaxDecayHeads = 256;
constexpr int kMaxOrder = 64;   // segments whose forward launch order is chosen

// One block of arguments for every forward-path kernel.  Sequence layout:
// head bh = b*H + h owns rows [bh*n, (bh+1)*n) of q, k ([.., d]) and v, o
// ([.., dv]).  The sequence is cut into `nseg` segments of `seg_len` tokens
// (the last may be shorter); a segment is cut into chunks of C tokens.
struct FwdParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    int BH, H, n;
    int seg_len;      // tokens per segment (a multiple of the chunk)
    int nseg;         // segments per head
    int nreal;        // summarised segments per head: nseg - 1
    int leaf_fold;    // no up-sweep: segment s folds leaves 0 .. s-1 one by one
    int ratio;        // divide by the masked denominator
    float *ws;        // workspace, see below (unused when nseg == 1)
    const float *state_in;   // [BH][state floats] or null
    float *state_out;        // [BH][state floats] or null
    void *z_out;             // rows of the first chained pass, or null: HLA-2 z_t = S_t q_t
                             // ([BH][n][D]), AHLA y_t = P_t^T q_t ([BH][n][DV]); T
    float gamma[kMaxDecayHeads];  // decay of head h (1 when none)
    short seg_order[kMaxOrder];    // forward: segment run by rank r (nseg <= kMaxOrder)
};

// Decay of head index h (= bh % H).  Only the first kMaxDecayHeads entries of
// a gamma array exist; a per-head decay is accepted only for H up to that,
// and without one every entry is 1, so clamping the index keeps the read
// inside the array for any H.
__host__ __device__ inline int gamma_slot(int bh, int H) {
    const int h = bh % H;
    return h < kMaxDecayHeads ? h : kMaxDecayHeads - 1;
}

// Forward workgroup L of the 1-D grid of nseg * BH: heads vary fastest, so
// consecutive workgroups -- dealt to different XCDs -- share one segment
// rank, and every XCD gets every segment; rank r runs segment seg_order[r]
// (ranks ordered so the workgroups that meet on a compute unit pair a costly
// prefix with a cheap one).
__device__ inline void forward_slot(const FwdParams &p, int L, int *seg, int *bh) {
    const int r = L / p.BH;
    *bh = L - r * p.BH;
    *seg = p.nseg <= kMaxOrder ? p.seg_order[r] : r;
}

// Segment summary, fp32, D x D then D x DV then D x DV then D then D:
//            X        Y        N      y     nv
//   HLA-2:   S        C        W      m     u      (W = S^K C^QV - G, u = S^K m^Q - h)
//   AHLA :   M        P        E      mK    nk     (M = sum k q^T)
//
// Workspace (fp32): the leaves, then the internal nodes of the scan's
// up-sweep tree.  Node (b, m) covers segments [m 2^b, (m+1) 2^b - 1]; only
// nodes ending below nreal exist, so level b has nreal >> b of them.  Leaf
// (0, s) is the summary of segment s, at ws + (bh*nreal + s) * summary_floats;
// internal node (b >= 1, m) is at ws + (BH*nreal + bh*nreal + node_index(b, m))
// * summary_floats.
__host__ __device__ constexpr int summary_floats(int D, int DV) { return D * D + 2 * D * DV + 2 * D; }
__host__ __device__ constexpr int hla2_state_floats(int D, int DV) { return D * D + D * DV + D; }
__host__ __device__ constexpr int ahla_state_floats(int D, int DV) { return 2 * D * DV + 2 * D; }
// third order: [B*H][D*DV] P^KV blocks, then [B*H][hla2_state_floats] the
// second-order state of (q, k, y), y = P^T q
__host__ __device__ constexpr int hla3_state_floats(int D, int DV) { return D * DV + hla2_state_floats(D, DV); }

template <int D, int DV>
struct SumOfs {
    static constexpr int X = 0, Y = D * D, N = D * D + D * DV, y = D * D + 2 * D * DV,
                         nv = D * D + 2 * D * DV + D;
};

// index of internal node (b >= 1, m) among its head's internal nodes
__host__ __device__ inline int node_index(int b, int m, int nreal) {
    int off = 0;
    for (int l = 1; l < b; ++l) off += nreal >> l;
    return off + m;
}
__host__ __device__ inline size_t node_offset(int bh, int b, int m, int BH, int nreal, int sumf) {
    const size_t slot = b == 0 ? (size_t)bh * nreal + m
                               : (size_t)BH * nreal + (size_t)bh * nreal + node_index(b, m, nreal);
    return slot * (size_t)sumf;
}

// Arguments of one chunked first-order linear-attention pass (la_kernels.h):
//   out_t = add_t + sum_{s <= t} g^(t-s) (a_t . b_s) c_s,
// over the reversed sequence when `reverse` is set.
struct LaParams {
    const void *a;      // [BH][n][D] queries of this pass
    const void *b;      // [BH][n][D] keys
    const void *c;      // [BH][n][D] values
    const void *add;    // [BH][n][D] added to the output, or null (may alias out)
    void *out;          // [BH][n][D]
    const void *a2;     // [BH][n][D] queries of the second output (DUAL form), else null
    void *out2;         // [BH][n][D] second output (DUAL form), else null
    const void *add2;   // [BH][n][D] added to out2, or null (may alias out2)
    float *sums;        // [BH][nseg-1][D*D] segment states (nseg > 1)
    int BH, H, n;
    int seg_len;        // tokens per segment, a multiple of the chunk
    int nseg;
    int reverse;        // run the sequence backwards (anti-causal pass)
    const float *state_in;   // head bh's D*D state before token 0 at state_in + bh*state_stride, or null
    float *state_out;        // the state after token n-1, same layout, or null
    float *state_out2;       // a second copy of it, same layout, or null
    long state_stride;       // floats between heads' states (0: D*D)
    float gamma[kMaxDecayHeads];   // decay of head h for this pass
};

// Gradient of the per-head decays of HLA-2 (la_kernels.h,
// decay_grad_rows_kernel and decay_grad_final_kernel).  With Z = LA_g(Q, K, K)
// and dZ the full gradient reaching Z, differentiating every g^(t-s) factor of
// the two chained passes gives
//     g_h dL/dg_h = sum_{b, t} (t - c) (2 q_t . dq_t - 3 z_t . dz_t - k_t . dk_t / 2)
// for any constant c (the sum without the weight is zero); c = (n - 1) / 2
// keeps the terms small.  The same sum holds for the ratio form.
constexpr int kDecayGradBlocks = 64;   // most row workgroups per head
struct DecayGradParams {
    const void *q, *k, *z, *dq, *dk, *dz;   // [BH][n][D]
    double *partial;                        // [BH][nblk]
    float *dgamma;                          // [H] out
    long n;
    int BH, H, nblk;
    float gamma[kMaxDecayHeads];            // decay of head h (1 when none)
};

// Row-wise step of the ratio backward (la_kernels.h, ratio_prep_kernel).
struct RatioPrepParams {
    const void *q, *u, *num, *dout;   // [rows][D]
    void *g, *e1, *dq;                // [rows][D]
    long rows;
};

// Decode step arguments.
struct StepParams {
    const void *q;   // [BH][D]
    const void *k;   // [BH][D]
    const void *v;   // [BH][DV]
    void *o;         // [BH][DV]
    float *state;    // [BH][state floats]
    int BH, H;
    int ratio;
    float gamma[kMaxDecayHeads];
};

// StepParams' mode of the decode kernel
enum StepMode { kStepHla2 = 0, kStepAhla = 1, kStepHla3 = 2 };

}  // namespace hla
