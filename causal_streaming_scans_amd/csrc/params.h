// params.h -- kernel argument block and workspace layout (internal).
#pragma once

#include <stddef.h>

namespace hla {

constexpr int kMaxDecayHeads = 256;

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
    int ratio;        // divide by the masked denominator
    float *ws;        // workspace, see below (unused when nseg == 1)
    const float *state_in;   // [BH][state floats] or null
    float *state_out;        // [BH][state floats] or null
    float gamma[kMaxDecayHeads];  // decay of head h (1 when none)
};

// Segment summary, fp32, D x D then D x DV then D x DV then D then D:
//            X        Y        N      y     nv
//   HLA-2:   S        C        W      m     u      (W = S^K C^QV - G, u = S^K m^Q - h)
//   AHLA :   M        P        E      mK    nk     (M = sum k q^T)
//
// Workspace: for head bh, `nreal` summary slots, ws + (bh*nreal + slot) *
// summary_floats.  Slot s first receives the summary of segment s; the
// up-sweep of the scan then combines in place: node (b, m) covers segments
// [m 2^b, (m+1) 2^b - 1] and lives in the slot of its last segment, so a
// parent overwrites its right child, which nothing reads afterwards.  Only
// nodes ending below nreal are formed.
__host__ __device__ constexpr int summary_floats(int D, int DV) { return D * D + 2 * D * DV + 2 * D; }
__host__ __device__ constexpr int hla2_state_floats(int D, int DV) { return D * D + D * DV + D; }
__host__ __device__ constexpr int ahla_state_floats(int D, int DV) { return 2 * D * DV + 2 * D; }

template <int D, int DV>
struct SumOfs {
    static constexpr int X = 0, Y = D * D, N = D * D + D * DV, y = D * D + 2 * D * DV,
                         nv = D * D + 2 * D * DV + D;
};

__host__ __device__ inline size_t ws_node(int bh, int slot, int nreal, int sumf) {
    return ((size_t)bh * nreal + slot) * (size_t)sumf;
}
__host__ __device__ inline int node_slot(int b, int m) { return ((m + 1) << b) - 1; }

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

}  // namespace hla
