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
    int spad;         // nseg rounded up to a power of two
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
// Workspace: for head bh, the `spad` segment summaries ("e", written by the
// summary kernel, combined in place by the up-sweep) followed by the `spad`
// exclusive prefixes ("p", written by the down-sweep and read by the
// forward kernel):  ws + ((bh*2 + which) * spad + s) * summary_floats.
__host__ __device__ constexpr int summary_floats(int D, int DV) { return D * D + 2 * D * DV + 2 * D; }
__host__ __device__ constexpr int hla2_state_floats(int D, int DV) { return D * D + D * DV + D; }
__host__ __device__ constexpr int ahla_state_floats(int D, int DV) { return 2 * D * DV + 2 * D; }

__host__ __device__ inline size_t ws_elem(int bh, int which, int spad, int s, int sumf) {
    return ((size_t)(bh * 2 + which) * spad + s) * (size_t)sumf;
}

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
