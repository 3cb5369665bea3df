// hla_api.cpp -- the C ABI declared in include/hla.h.
//
// Validation runs first and touches no HIP API, so every error code below is
// reachable on a host without a GPU.  Then the forward pass enqueues, on the
// caller's stream:
//   stage 1: the segment-summary kernel over segments 0 .. nseg-2 (the last
//      segment's summary would only feed the total, which an exclusive scan
//      never uses);
//   stage 2: the up-sweep of the exclusive Blelloch scan over the summaries
//      (none with at most three summaries per head: each segment then
//      folds the leaves before it directly);
//   stage 3: the chunked forward kernel over every segment: each workgroup
//      first folds the caller's initial state and the up-sweep nodes left of
//      its segment into its carried state (the down-sweep's value for it).
// With a single segment only stage 3 runs, starting from state_in or zero.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/hla.h"
#include "launch.h"

using namespace hla;

namespace {

bool valid_variant(int v) { return v >= HLA_HLA2 && v <= HLA_HLA3_RATIO; }
bool is_hla3(int v) { return v == HLA_HLA3 || v == HLA_HLA3_RATIO; }
bool is_ahla(int v) { return v == HLA_AHLA || v == HLA_AHLA_RATIO; }
bool is_ratio(int v) {
    return v == HLA_HLA2_RATIO || v == HLA_AHLA_RATIO || v == HLA_HLA3_RATIO;
}
// third order as chained first-order passes: with a decay, or the ratio form
bool hla3_chain(int v, const float *gamma) {
    return v == HLA_HLA3_RATIO || (v == HLA_HLA3 && gamma != nullptr);
}

long ceil_div(long a, long b) { return (a + b - 1) / b; }

int effective_seg_chunks(int variant, int B, int H, int n, int d, int chunk, int seg_chunks) {
    return seg_chunks > 0 ? seg_chunks : hla_default_seg_chunks(variant, B, H, n, d, chunk);
}

long num_segments(int n, int chunk, int seg_chunks) {
    if (n <= 0) return 0;
    return ceil_div(n, (long)chunk * seg_chunks);
}

// Shared argument checks of forward and step.  Returns HLA_OK or the error.
hla_status check_common(int B, int H, int d, int dv, int dtype, int variant, const float *gamma) {
    if (dtype != HLA_F32 && dtype != HLA_BF16) return HLA_ERR_ARG;
    if (!valid_variant(variant)) return HLA_ERR_ARG;
    if (B < 1 || H < 1 || d < 1 || dv < 1) return HLA_ERR_SHAPE;
    if ((long)B * H > 65535) return HLA_ERR_UNSUPPORTED;
    if (gamma) {
        if (H > HLA_MAX_DECAY_HEADS) return HLA_ERR_UNSUPPORTED;
        for (int h = 0; h < H; ++h)
            if (!(gamma[h] > 0.f && gamma[h] <= 1.f)) return HLA_ERR_ARG;  // also rejects NaN
    }
    return HLA_OK;
}

// With at most three summarised segments per head the scan has no up-sweep:
// segment s folds leaves 0 .. s-1 one by one (at most three folds, two with
// cross terms), which costs less than the up-sweep's launch and its wait
// (four segments, B=8 H=16 n=4096 d=64: 88.0 -> 83.6 us per forward).
bool leaf_fold(int nreal) { return nreal <= 3; }

// Forward launch order of the segments (see forward_slot): by the number of
// nodes a segment folds into its prefix, costliest first over the
// first half of the ranks and cheapest first over the second half, so that
// the two workgroups a compute unit holds at once pair a costly prefix with
// a cheap one.
void fill_order(FwdParams *p) {
    const int n = p->nseg;
    if (n > kMaxOrder) return;
    int idx[kMaxOrder];
    for (int i = 0; i < n; ++i) idx[i] = i;
    for (int i = 1; i < n; ++i)   // insertion sort: fold count, then index, descending
        for (int j = i; j > 0; --j) {
            const int a = idx[j - 1], b = idx[j];
            const int ca = p->leaf_fold ? a : __builtin_popcount(a);
            const int cb = p->leaf_fold ? b : __builtin_popcount(b);
            if (ca > cb || (ca == cb && a > b)) break;
            idx[j - 1] = b;
            idx[j] = a;
        }
    const int h = (n + 1) / 2;
    for (int i = 0; i < h; ++i) p->seg_order[i] = (short)idx[i];
    for (int j = 0; j < n - h; ++j) p->seg_order[h + j] = (short)idx[n - 1 - j];
}

void fill_gamma(float *dst, const float *gamma, int H) {
    for (int h = 0; h < kMaxDecayHeads; ++h) dst[h] = (gamma && h < H) ? gamma[h] : 1.f;
}

// ------------------------------------------------------------ backward passes
//
// Each pass is one chunked linear-attention launch pair (la_kernels.h): a
// segment-state launch (unless `summaries` is false and `sums` already holds
// the states of the same b, c and decay) and the main launch, in the plain,
// SYM or DUAL form.  The pass lists below are in dependency order.

enum Form { PLAIN, SYM, DUAL };

struct Pass {
    const LaParams *base;   // sizes and decay (g or g^2)
    const void *a, *b, *c, *add;
    void *out;
    int rev;                // anti-causal: run backwards through memory
    Form form;
    float *sums;
    bool summaries;
    const void *a2;         // DUAL: second queries, output and addend
    void *out2;
    const void *add2;
};

// Inputs and gradients of one backward call; z: the forward's keyed queries
// (HLA-2 only), or null to recompute them.
struct Grads {
    const void *q, *k, *v, *dout;
    void *dq, *dk, *dv;
    const void *z = nullptr;
};

struct BwdCtx {
    LaLaunches la;
    LaParams p1, p2;        // decay g and g^2 (third order: g^3)
    bool p3_cube;
    float *sums_kk, *sums;  // K K^T states (first and last pass), the rest
    char *ws;
    size_t sums_bytes, tensor_bytes;
    long rows;
    hipStream_t s;

    // workspace tensor i of [B*H*n*d] after the segment states
    void *tensor(int i) const { return ws + 2 * sums_bytes + (size_t)i * tensor_bytes; }

    bool run(const Pass &ps) const {
        LaParams p = *ps.base;
        p.a = ps.a;
        p.b = ps.b;
        p.c = ps.c;
        p.add = ps.add;
        p.out = ps.out;
        p.a2 = ps.a2;
        p.out2 = ps.out2;
        p.add2 = ps.add2;
        p.reverse = ps.rev;
        p.sums = ps.sums;
        const LaLaunch fn = ps.form == SYM ? la.sym : ps.form == DUAL ? la.dual : la.plain;
        return fn(p, s, ps.summaries) == hipSuccess;
    }
    // the segment-state launch of a plain pass alone
    static LaParams states_params(const Pass &ps) {
        LaParams p = *ps.base;
        p.b = ps.b;
        p.c = ps.c;
        p.reverse = ps.rev;
        p.sums = ps.sums;
        return p;
    }
    bool states(const Pass &ps) const { return la.states(states_params(ps), s) == hipSuccess; }
    // those of three plain passes in one launch
    bool states3(const Pass &a, const Pass &b, const Pass &c3) const {
        const LaParams p3[3] = {states_params(a), states_params(b), states_params(c3)};
        return la.states3(p3, s) == hipSuccess;
    }
    hla_status run_all(const Pass *ps, int count) const {
        for (int i = 0; i < count; ++i)
            if (!run(ps[i])) return HLA_ERR_DEVICE;
        return HLA_OK;
    }
};

// HLA-2: Z = LA_g(Q, K, K), O = LA_{g^2}(Q, Z, V) (Z, dZ in tensors 0, 1;
// Z is the caller's when x.z is given).
hla_status backward_hla2(const BwdCtx &c, const Grads &x) {
    void *Z = x.z ? const_cast<void *>(x.z) : c.tensor(0), *dZ = c.tensor(1);
    const Pass passes[5] = {
        // Z  = LA_g(Q, K, K)
        {&c.p1, x.q, x.k, x.k, nullptr, Z, 0, PLAIN, c.sums_kk, true, nullptr, nullptr, nullptr},
        // dQ = LA_g2(dO, V, Z)
        {&c.p2, x.dout, x.v, Z, nullptr, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // dZ = RLA_g2(V, dO, Q) and dV = RLA_g2(Z, Q, dO): one state, sum dO Q^T
        {&c.p2, x.v, x.dout, x.q, nullptr, dZ, 1, DUAL, c.sums, true, Z, x.dv, nullptr},
        // dK = RLA_g(K, dZ, Q) + RLA_g(K, Q, dZ)
        {&c.p1, x.k, dZ, x.q, nullptr, x.dk, 1, SYM, c.sums, true, nullptr, nullptr, nullptr},
        // dQ += LA_g(dZ, K, K), with the segment states of the first pass
        {&c.p1, dZ, x.k, x.k, x.dq, x.dq, 0, PLAIN, c.sums_kk, false, nullptr, nullptr, nullptr},
    };
    if (!x.z) return c.run_all(passes, 5);
    // Z from the forward: of the first pass only its segment states, which
    // the last pass reads.  Those, and the states of the next two passes,
    // need only the inputs and Z: one launch forms all three, the third
    // into the unused Z slot when it holds them (at d = 128 with very short
    // segments it may not: three launches then)
    if (c.sums_bytes > c.tensor_bytes) {
        if (!c.states(passes[0])) return HLA_ERR_DEVICE;
        return c.run_all(passes + 1, 4);
    }
    Pass dq = passes[1], dzv = passes[2];
    dq.summaries = false;
    dzv.summaries = false;
    dzv.sums = reinterpret_cast<float *>(c.tensor(0));
    if (!c.states3(passes[0], dq, dzv)) return HLA_ERR_DEVICE;
    const Pass rest[4] = {dq, dzv, passes[3], passes[4]};
    return c.run_all(rest, 4);
}

// AHLA: Y = LA(Q, K, V), O = LA(Q, K, Y), no decay (Y, dY in tensors 0, 1;
// Y is the caller's when x.z is given).
hla_status backward_ahla(const BwdCtx &c, const Grads &x) {
    void *Y = x.z ? const_cast<void *>(x.z) : c.tensor(0), *dY = c.tensor(1);
    const Pass passes[5] = {
        // Y  = LA(Q, K, V)
        {&c.p1, x.q, x.k, x.v, nullptr, Y, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // dQ = LA(dO, Y, K)
        {&c.p1, x.dout, Y, x.k, nullptr, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // dY = RLA(K, Q, dO) and dK = RLA(Y, dO, Q): one state, sum Q dO^T
        {&c.p1, x.k, x.q, x.dout, nullptr, dY, 1, DUAL, c.sums, true, Y, x.dk, nullptr},
        // dV = RLA(K, Q, dY) and dK += RLA(V, dY, Q): one state, sum Q dY^T
        {&c.p1, x.k, x.q, dY, nullptr, x.dv, 1, DUAL, c.sums, true, x.v, x.dk, x.dk},
        // dQ += LA(dY, V, K)
        {&c.p1, dY, x.v, x.k, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
    };
    // Y from the forward: the first pass is not needed at all (no later
    // pass reads its segment states)
    return x.z ? c.run_all(passes + 1, 4) : c.run_all(passes, 5);
}

// Ratio HLA-2, o = num / den with den the v == 1 sum.  With G = dO / den and
// e = -(dO . o) / den per row, the gradient is that of num with upstream G,
// plus den's: dq += e_t u_t, u = LA_g2(ONE1, ONE1, Z) (u_t = sum_j
// g^(2(t-j)) z_j), and dZ += RLA_g2(ONE1, E1, Q) (sum_{t>=j} g^(2(t-j)) e_t q_t),
// where ONE1 has rows (1, 0, ..., 0) and E1 rows (e_t, 0, ..., 0).  den is
// q_t . u_t and num = LA_g2(Q, Z, V); u lives in dv and num in dZ's buffer
// until the passes that overwrite them.  Tensors: Z, dZ, G, E1, ONE1.
hla_status backward_hla2_ratio(const BwdCtx &c, const Grads &x) {
    void *Z = c.tensor(0), *dZ = c.tensor(1), *G = c.tensor(2), *E1 = c.tensor(3),
         *ONE1 = c.tensor(4);
    if (c.la.unit_column(ONE1, c.rows, c.s) != hipSuccess) return HLA_ERR_DEVICE;
    const Pass pre[3] = {
        // Z  = LA_g(Q, K, K)
        {&c.p1, x.q, x.k, x.k, nullptr, Z, 0, PLAIN, c.sums_kk, true, nullptr, nullptr, nullptr},
        // u  = LA_g2(ONE1, ONE1, Z)
        {&c.p2, ONE1, ONE1, Z, nullptr, x.dv, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // num = LA_g2(Q, Z, V)
        {&c.p2, x.q, Z, x.v, nullptr, dZ, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
    };
    hla_status st = c.run_all(pre, 3);
    if (st != HLA_OK) return st;
    const RatioPrepParams rp{x.q, x.dv, dZ, x.dout, G, E1, x.dq, c.rows};
    if (c.la.ratio_prep(rp, c.s) != hipSuccess) return HLA_ERR_DEVICE;
    const Pass post[5] = {
        // dQ = e u + LA_g2(G, V, Z)
        {&c.p2, G, x.v, Z, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // dZ = RLA_g2(V, G, Q) and dV = RLA_g2(Z, Q, G)
        {&c.p2, x.v, G, x.q, nullptr, dZ, 1, DUAL, c.sums, true, Z, x.dv, nullptr},
        // dZ += RLA_g2(ONE1, E1, Q)
        {&c.p2, ONE1, E1, x.q, dZ, dZ, 1, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // dK = RLA_g(K, dZ, Q) + RLA_g(K, Q, dZ)
        {&c.p1, x.k, dZ, x.q, nullptr, x.dk, 1, SYM, c.sums, true, nullptr, nullptr, nullptr},
        // dQ += LA_g(dZ, K, K), with the segment states of the first pass
        {&c.p1, dZ, x.k, x.k, x.dq, x.dq, 0, PLAIN, c.sums_kk, false, nullptr, nullptr, nullptr},
    };
    return c.run_all(post, 5);
}

// Ratio AHLA: num = LA(Q, K, Y), den = first column of LA(Q, K, Y1) with
// Y = LA(Q, K, V), Y1 = LA(Q, K, ONE1).  The gradient is the AHLA chain with
// upstream G on values V plus the AHLA chain with upstream E1 on values ONE1
// (whose value gradient is dropped).  Tensors: Y, dY, G, E1, ONE1, Y1, dY1;
// num lives in dY's buffer and den in dY1's until those are written.
hla_status backward_ahla_ratio(const BwdCtx &c, const Grads &x) {
    void *Y = c.tensor(0), *dY = c.tensor(1), *G = c.tensor(2), *E1 = c.tensor(3),
         *ONE1 = c.tensor(4), *Y1 = c.tensor(5), *dY1 = c.tensor(6);
    if (c.la.unit_column(ONE1, c.rows, c.s) != hipSuccess) return HLA_ERR_DEVICE;
    const Pass pre[4] = {
        {&c.p1, x.q, x.k, x.v, nullptr, Y, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},    // Y
        {&c.p1, x.q, x.k, ONE1, nullptr, Y1, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},  // Y1
        {&c.p1, x.q, x.k, Y, nullptr, dY, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},     // num
        {&c.p1, x.q, x.k, Y1, nullptr, dY1, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},   // den
    };
    hla_status st = c.run_all(pre, 4);
    if (st != HLA_OK) return st;
    // den = ONE1_t . DEN_t, the first column; the row kernel's e u output is
    // not used here and goes to dv, which a later pass writes
    const RatioPrepParams rp{ONE1, dY1, dY, x.dout, G, E1, x.dv, c.rows};
    if (c.la.ratio_prep(rp, c.s) != hipSuccess) return HLA_ERR_DEVICE;
    const Pass post[8] = {
        // upstream G, values V
        {&c.p1, G, Y, x.k, nullptr, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        {&c.p1, x.k, x.q, G, nullptr, dY, 1, DUAL, c.sums, true, Y, x.dk, nullptr},
        {&c.p1, x.k, x.q, dY, nullptr, x.dv, 1, DUAL, c.sums, true, x.v, x.dk, x.dk},
        {&c.p1, dY, x.v, x.k, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // upstream E1, values ONE1
        {&c.p1, E1, Y1, x.k, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        {&c.p1, x.k, x.q, E1, nullptr, dY1, 1, DUAL, c.sums, true, Y1, x.dk, x.dk},
        {&c.p1, ONE1, dY1, x.q, x.dk, x.dk, 1, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        {&c.p1, dY1, ONE1, x.k, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
    };
    return c.run_all(post, 8);
}

// Third order: Y = LA_g(Q, K, V), Z = LA_g(Q, K, K), O = LA_{g^3}(Q, Z, Y)
// (p1 carries g, p2 here g^3).  The ratio form adds the unit-value chain
// Y1 = LA_g(Q, K, ONE1), DEN = LA_{g^3}(Q, Z, Y1), o = O / DEN[:, 0]: its
// upstream is G = dO / den on O and E1 = (e, 0, ..., 0) on DEN.  Through O:
// dQ = LA(G, Y, Z), dZ = RLA(Y, G, Q), dY = RLA(Z, Q, G) (dZ and dY one DUAL
// pass), and the same with E1 and Y1 for DEN; through Z: dK = RLA(K, dZ, Q) +
// RLA(K, Q, dZ) (SYM), dQ += LA(dZ, K, K); through Y: dQ += LA(dY, V, K),
// dV = RLA(K, Q, dY) and dK += RLA(V, dY, Q) (DUAL); through Y1:
// dQ += LA(dY1, ONE1, K), dK += RLA(ONE1, dY1, Q).  Tensors: Y, Z, dZ, dY
// and for the ratio form G, E1, ONE1, Y1, dY1, NUM, DEN, a spare.
hla_status backward_hla3(const BwdCtx &c, const Grads &x, bool ratio) {
    void *Y = c.tensor(0), *Z = c.tensor(1), *dZ = c.tensor(2), *dY = c.tensor(3);
    const Pass fwd[2] = {
        {&c.p1, x.q, x.k, x.v, nullptr, Y, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        {&c.p1, x.q, x.k, x.k, nullptr, Z, 0, PLAIN, c.sums_kk, true, nullptr, nullptr, nullptr},
    };
    hla_status st = c.run_all(fwd, 2);
    if (st != HLA_OK) return st;
    const void *up = x.dout;
    void *G = nullptr, *E1 = nullptr, *ONE1 = nullptr, *Y1 = nullptr, *dY1 = nullptr;
    if (ratio) {
        G = c.tensor(4);
        E1 = c.tensor(5);
        ONE1 = c.tensor(6);
        Y1 = c.tensor(7);
        dY1 = c.tensor(8);
        void *NUM = c.tensor(9), *DEN = c.tensor(10), *spare = c.tensor(11);
        if (c.la.unit_column(ONE1, c.rows, c.s) != hipSuccess) return HLA_ERR_DEVICE;
        const Pass pre[3] = {
            {&c.p1, x.q, x.k, ONE1, nullptr, Y1, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
            {&c.p2, x.q, Z, Y, nullptr, NUM, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
            {&c.p2, x.q, Z, Y1, nullptr, DEN, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        };
        st = c.run_all(pre, 3);
        if (st != HLA_OK) return st;
        // den = ONE1 . DEN (its first column); the e u output is not used here
        const RatioPrepParams rp{ONE1, DEN, NUM, x.dout, G, E1, spare, c.rows};
        if (c.la.ratio_prep(rp, c.s) != hipSuccess) return HLA_ERR_DEVICE;
        up = G;
    }
    const Pass through_o[2] = {
        // dQ = LA(G, Y, Z)
        {&c.p2, up, Y, Z, nullptr, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // dZ = RLA(Y, G, Q) and dY = RLA(Z, Q, G)
        {&c.p2, Y, up, x.q, nullptr, dZ, 1, DUAL, c.sums, true, Z, dY, nullptr},
    };
    st = c.run_all(through_o, 2);
    if (st != HLA_OK) return st;
    if (ratio) {
        const Pass through_den[2] = {
            {&c.p2, E1, Y1, Z, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
            {&c.p2, Y1, E1, x.q, dZ, dZ, 1, DUAL, c.sums, true, Z, dY1, nullptr},
        };
        st = c.run_all(through_den, 2);
        if (st != HLA_OK) return st;
    }
    const Pass rest[4] = {
        // dK = RLA(K, dZ, Q) + RLA(K, Q, dZ)
        {&c.p1, x.k, dZ, x.q, nullptr, x.dk, 1, SYM, c.sums, true, nullptr, nullptr, nullptr},
        // dQ += LA(dZ, K, K), with the segment states of the Z pass
        {&c.p1, dZ, x.k, x.k, x.dq, x.dq, 0, PLAIN, c.sums_kk, false, nullptr, nullptr, nullptr},
        // dQ += LA(dY, V, K)
        {&c.p1, dY, x.v, x.k, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        // dV = RLA(K, Q, dY) and dK += RLA(V, dY, Q)
        {&c.p1, x.k, x.q, dY, nullptr, x.dv, 1, DUAL, c.sums, true, x.v, x.dk, x.dk},
    };
    st = c.run_all(rest, 4);
    if (st != HLA_OK || !ratio) return st;
    const Pass unit[2] = {
        // dQ += LA(dY1, ONE1, K) ; dK += RLA(ONE1, dY1, Q)
        {&c.p1, dY1, ONE1, x.k, x.dq, x.dq, 0, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
        {&c.p1, ONE1, dY1, x.q, x.dk, x.dk, 1, PLAIN, c.sums, true, nullptr, nullptr, nullptr},
    };
    return c.run_all(unit, 2);
}

// dL/dg_h from the tensors the HLA-2 passes leave behind (DecayGradParams):
// x's q, k, dq, dk in the pass dtype, Z and dZ in workspace tensors 0 and 1.
hla_status decay_gradient(const BwdCtx &c, const Grads &x, int H, int n, int d, float *dgamma,
                          void *partial) {
    DecayGradParams p;
    memset(&p, 0, sizeof(p));
    p.q = x.q;
    p.k = x.k;
    p.z = c.tensor(0);
    p.dq = x.dq;
    p.dk = x.dk;
    p.dz = c.tensor(1);
    p.partial = static_cast<double *>(partial);
    p.dgamma = dgamma;
    p.n = n;
    p.BH = c.p1.BH;
    p.H = H;
    // rows per workgroup step: 4 waves of 64 / (d / N) rows, N = the values
    // in 16 bytes; about 1024 workgroups in all, at most kDecayGradBlocks
    // per head
    const int per16 = 16 / (int)(c.tensor_bytes / ((size_t)c.rows * d));
    const long rpb = 4L * (64 / (d / per16));
    long nblk = ceil_div(1024, p.BH);
    if (nblk > kDecayGradBlocks) nblk = kDecayGradBlocks;
    if (nblk > ceil_div(n, rpb)) nblk = ceil_div(n, rpb);
    p.nblk = (int)nblk;
    memcpy(p.gamma, c.p1.gamma, sizeof(p.gamma));
    return c.la.decay_grad(p, c.s) == hipSuccess ? HLA_OK : HLA_ERR_DEVICE;
}

}  // namespace

extern "C" {

size_t hla_state_floats(int variant, int d, int dv) {
    if (!valid_variant(variant) || d < 1 || dv < 1) return 0;
    if (variant == HLA_HLA3_RATIO) return 2 * (size_t)hla3_state_floats(d, dv);
    if (is_hla3(variant)) return (size_t)hla3_state_floats(d, dv);
    return is_ahla(variant) ? (size_t)ahla_state_floats(d, dv) : (size_t)hla2_state_floats(d, dv);
}

int hla_default_seg_chunks(int variant, int B, int H, int n, int d, int chunk) {
    (void)variant;
    if (B < 1 || H < 1 || n < 1 || d < 1 || chunk < 1) return 1;
    const long nch = ceil_div(n, chunk);
    const long bh = (long)B * H;
    // Enough segments to give the 256 compute units about two workgroups
    // each, but no segment shorter than 8 chunks: short segments add summary
    // work and scan depth without adding useful parallelism.  At d >= 128 a
    // summary (and each combine of the up-sweep) is O(d^2 dv) and costs as
    // much as several chunks of the forward, so one workgroup per compute
    // unit is the better trade.
    const long target_wg = d >= 128 ? 256 : 512;
    long nseg = ceil_div(target_wg, bh);
    if (nseg <= 1) return (int)nch;
    long g = ceil_div(nch, nseg);
    if (g < 8) g = 8;
    if (g > nch) g = nch;
    return (int)g;
}

size_t hla_workspace_bytes(int variant, int B, int H, int n, int d, int dv, int chunk,
                           int seg_chunks) {
    if (!valid_variant(variant) || B < 1 || H < 1 || n < 1 || d < 1 || dv < 1 || chunk < 1 ||
        seg_chunks < 0)
        return 0;
    const int g = effective_seg_chunks(variant, B, H, n, d, chunk, seg_chunks);
    const long nseg = num_segments(n, chunk, g);
    // leaves, then internal nodes of the up-sweep (fewer than nreal per head)
    const size_t scan = nseg <= 1 ? 0
        : 2 * (size_t)B * H * (size_t)(nseg - 1) * (size_t)summary_floats(d, dv) * sizeof(float);
    if (!is_hla3(variant)) return scan;
    // third order: the segment states of its first-order passes, then
    // [B*H][n][d] fp32 tensors: Y and Z of the decayed chain (the undecayed
    // form uses the first for Y); the ratio form also widened q, k, v, the
    // unit rows, Y1, the numerator and the denominator
    const long nseg_la = num_segments(n, kLaChunk, hla_backward_default_seg_chunks(B, H, n));
    const size_t sums = (size_t)B * H * (size_t)(nseg_la - 1) * d * dv * sizeof(float);
    const size_t tensor = (size_t)B * H * n * dv * sizeof(float);
    return scan + sums + (variant == HLA_HLA3_RATIO ? 9 : 2) * tensor;
}

// The first-order pass of the third-order variant, Y = LA(Q, K, V), run
// before the second-order stages consume (Q, K, Y).
struct Hla3Pass {
    LaLaunches la;
    LaParams lp;
    // the chained form (a decay, or the ratio form): passes of decay g (p1)
    // and g^3 (p3) over the tensors in the workspace
    bool chain, ratio, widen;
    LaLaunches lac;
    LaParams p1, p3;
    const void *q, *k, *v;
    void *o;
    char *tensors;
    size_t tensor_bytes;
    long rows;
    int d;
    const float *state_in;
    float *state_out;
    size_t state_count;     // floats of state_out
};

// State views of the third-order layout (per head bh): the P^KV block at
// base + bh*d*dv, then the second-order block [S | W | u] at
// base + BH*d*dv + bh*(d*d + d*dv + d); the ratio form's unit-value chain
// repeats that layout after it.
// (one function for both the input and the output state: the result is
// handed back as writable, the caller keeps the input's constness)
static float *hla3_view(const float *base, int BH, int d, int part, int chain) {
    if (!base) return nullptr;
    const size_t one = (size_t)BH * hla3_state_floats(d, d);
    float *b = const_cast<float *>(base) + (size_t)chain * one;
    if (part == 0) return b;                                  // P
    b += (size_t)BH * d * d;
    return part == 1 ? b : b + (size_t)d * d;                 // S, W
}

// Third order with a decay or in the ratio form:
//   Y = LA_g(Q, K, V),  Z = LA_g(Q, K, K),  O = LA_{g^3}(Q, Z, Y)
// (keys z_m = S_m q_m and values y_m = P_m^T q_m, each decayed to m, meet
// with g^(3(t-m))); the ratio form runs the value chain again on unit rows
// ONE1, Y1 = LA_g(Q, K, ONE1), DEN = LA_{g^3}(Q, Z, Y1), in fp32, and
// divides.  Tensors: [qw, kw, vw (widened bf16 inputs),] Y, Z[, ONE1, Y1,
// O, DEN].
static hla_status run_hla3_chain(const Hla3Pass &x, hipStream_t s) {
    const LaLaunches &la = x.lac;
    auto t = [&](int i) { return static_cast<void *>(x.tensors + (size_t)i * x.tensor_bytes); };
    const void *q = x.q, *k = x.k, *v = x.v;
    const long count = x.rows * x.d;
    if (x.widen) {
        const void *src[3] = {x.q, x.k, x.v};
        for (int i = 0; i < 3; ++i)
            if (launch_convert(src[i], t(i), count, true, s) != hipSuccess) return HLA_ERR_DEVICE;
        q = t(0);
        k = t(1);
        v = t(2);
    }
    const int base = x.ratio ? 3 : 0;
    void *Y = t(base), *Z = t(base + 1);
    void *O = x.ratio ? t(base + 4) : x.o;
    const int BH = x.p1.BH, d = x.d;
    const long hla2_stride = hla2_state_floats(d, d);
    // the u slots are not used by third order: the whole state starts at zero
    if (x.state_out && launch_copy_or_zero(nullptr, x.state_out, x.state_count, s) != hipSuccess)
        return HLA_ERR_DEVICE;
    auto pass = [&](const LaParams &base_p, const void *a, const void *b, const void *c, void *out,
                    int part, int chain, bool second_copy) {
        LaParams p = base_p;
        p.a = a;
        p.b = b;
        p.c = c;
        p.out = out;
        p.state_stride = part == 0 ? 0 : hla2_stride;
        p.state_in = hla3_view(x.state_in, BH, d, part, chain);
        p.state_out = hla3_view(x.state_out, BH, d, part, chain);
        p.state_out2 = second_copy ? hla3_view(x.state_out, BH, d, part, 1) : nullptr;
        return la.plain(p, s, true) == hipSuccess;
    };
    if (!pass(x.p1, q, k, v, Y, 0, 0, false)) return HLA_ERR_DEVICE;           // Y, P
    if (!pass(x.p1, q, k, k, Z, 1, 0, x.ratio)) return HLA_ERR_DEVICE;         // Z, S
    if (!pass(x.p3, q, Z, Y, O, 2, 0, false)) return HLA_ERR_DEVICE;           // O, W
    if (!x.ratio) return HLA_OK;
    void *ONE1 = t(base + 2), *Y1 = t(base + 3), *DEN = t(base + 5);
    if (la.unit_column(ONE1, x.rows, s) != hipSuccess) return HLA_ERR_DEVICE;
    if (!pass(x.p1, q, k, ONE1, Y1, 0, 1, false)) return HLA_ERR_DEVICE;       // Y1, P of ONE1
    if (!pass(x.p3, q, Z, Y1, DEN, 2, 1, false)) return HLA_ERR_DEVICE;        // DEN, its W
    return launch_divide_rows(static_cast<const float *>(O), static_cast<const float *>(DEN),
                              x.o, x.rows, d, !x.widen ? false : true, s) == hipSuccess
               ? HLA_OK : HLA_ERR_DEVICE;
}

// Validate, pick the kernels and fill the argument block; shared by
// hla_forward and hla_forward_stage.
static hla_status prepare_forward(const void *q, const void *k, const void *v, void *o, int B,
                                  int H, int n, int d, int dv, int dtype, int variant,
                                  const float *gamma_host, int chunk, int seg_chunks,
                                  const float *state_in, float *state_out, void *workspace,
                                  size_t workspace_bytes, FwdKernels *kern, FwdParams *p,
                                  Hla3Pass *x3) {
    hla_status st = check_common(B, H, d, dv, dtype, variant, gamma_host);
    if (st != HLA_OK) return st;
    if (n < 0) return HLA_ERR_SHAPE;
    if (chunk < 0 || seg_chunks < 0) return HLA_ERR_ARG;
    if (n > 0 && (!q || !k || !v || !o)) return HLA_ERR_NULL;
    if (state_in && state_out && state_in == state_out) return HLA_ERR_ARG;
    if (!lookup_forward(dtype, is_ahla(variant), d, dv, chunk, gamma_host != nullptr, kern))
        return HLA_ERR_UNSUPPORTED;
    if (is_hla3(variant) && (d != dv || !lookup_la(dtype, d, &x3->la))) return HLA_ERR_UNSUPPORTED;
    x3->chain = hla3_chain(variant, gamma_host);
    if (x3->chain && !lookup_la(variant == HLA_HLA3_RATIO ? HLA_F32 : dtype, d, &x3->lac))
        return HLA_ERR_UNSUPPORTED;
    const int g = effective_seg_chunks(variant, B, H, n, d, chunk, seg_chunks);
    if ((long)chunk * g > INT32_MAX / 2) return HLA_ERR_UNSUPPORTED;
    const long nseg = num_segments(n, chunk, g);
    if (nseg > INT32_MAX / 4) return HLA_ERR_UNSUPPORTED;
    // one-dimensional grids: the forward's nseg*B*H workgroups, the up-sweep's
    // four (dv >= 128: eight) column slices of (nseg-1)/2*B*H combines
    if (nseg * B * H > (dv >= 128 ? INT32_MAX / 4 : INT32_MAX / 2)) return HLA_ERR_UNSUPPORTED;
    const size_t need = hla_workspace_bytes(variant, B, H, n, d, dv, chunk, g);
    if (need > 0) {
        if (!workspace) return HLA_ERR_NULL;
        if (workspace_bytes < need) return HLA_ERR_WORKSPACE;
    }
    memset(p, 0, sizeof(*p));
    p->q = q;
    p->k = k;
    p->v = v;
    p->o = o;
    p->BH = B * H;
    p->H = H;
    p->n = n;
    p->seg_len = chunk * g;
    p->nseg = (int)nseg;
    p->nreal = nseg > 1 ? (int)(nseg - 1) : 0;
    p->leaf_fold = leaf_fold(p->nreal) ? 1 : 0;
    p->ratio = is_ratio(variant) ? 1 : 0;
    p->ws = static_cast<float *>(workspace);
    p->state_in = state_in;
    p->state_out = state_out;
    fill_gamma(p->gamma, gamma_host, H);
    fill_order(p);
    if (is_hla3(variant)) {
        // after the scan's part of the workspace: the first-order passes'
        // segment states, then the tensors (Y first, which the second-order
        // stages of the undecayed form read as their values)
        const size_t scan = nseg <= 1 ? 0
            : 2 * (size_t)B * H * (size_t)(nseg - 1) * (size_t)summary_floats(d, dv) * sizeof(float);
        const int g_la = hla_backward_default_seg_chunks(B, H, n);
        const long nseg_la = num_segments(n, kLaChunk, g_la);
        char *sums = static_cast<char *>(workspace) + scan;
        char *tensors = sums + (size_t)B * H * (size_t)(nseg_la > 0 ? nseg_la - 1 : 0) * d * dv * sizeof(float);
        char *Y = tensors;
        LaParams &lp = x3->lp;
        memset(&lp, 0, sizeof(lp));
        lp.a = q;
        lp.b = k;
        lp.c = v;
        lp.out = Y;
        lp.sums = reinterpret_cast<float *>(sums);
        lp.BH = B * H;
        lp.H = H;
        lp.n = n;
        lp.seg_len = kLaChunk * g_la;
        lp.nseg = (int)nseg_la;
        fill_gamma(lp.gamma, nullptr, H);
        if (x3->chain) {
            x3->ratio = variant == HLA_HLA3_RATIO;
            x3->widen = x3->ratio && dtype == HLA_BF16;
            x3->p1 = lp;
            fill_gamma(x3->p1.gamma, gamma_host, H);
            x3->p3 = x3->p1;
            for (int h = 0; h < kMaxDecayHeads; ++h)
                x3->p3.gamma[h] = x3->p1.gamma[h] * x3->p1.gamma[h] * x3->p1.gamma[h];
            x3->q = q;
            x3->k = k;
            x3->v = v;
            x3->o = o;
            x3->tensors = tensors;
            x3->tensor_bytes = (size_t)B * H * n * dv * sizeof(float);
            x3->rows = (long)B * H * n;
            x3->d = d;
            x3->state_in = state_in;
            x3->state_out = state_out;
            x3->state_count = (size_t)B * H * hla_state_floats(variant, d, dv);
            return HLA_OK;
        }
        p->v = Y;
        // state: the P^KV blocks of all heads, then the second-order states
        const size_t pkv = (size_t)B * H * d * dv;
        lp.state_in = state_in;
        lp.state_out = state_out;
        p->state_in = state_in ? state_in + pkv : nullptr;
        p->state_out = state_out ? state_out + pkv : nullptr;
    }
    return HLA_OK;
}

// one stage of the forward pass (1 = summaries, 2 = up-sweep, 3 = chunked forward)
static hla_status run_stage(int stage, const FwdKernels &kern, const FwdParams &p, int variant,
                            int d, int dv, const Hla3Pass &x3, hipStream_t s) {
    if (p.n == 0) {
        // no tokens: the state passes through unchanged (done by the last stage)
        if (stage == 3 && p.state_out) {
            const size_t cnt = (size_t)p.BH * hla_state_floats(variant, d, dv);
            if (launch_copy_or_zero(p.state_in, p.state_out, cnt, s) != hipSuccess)
                return HLA_ERR_DEVICE;
        }
        return HLA_OK;
    }
    hipError_t e = hipSuccess;
    if (is_hla3(variant) && x3.chain) return stage == 3 ? run_hla3_chain(x3, s) : HLA_OK;
    if (stage == 1 && is_hla3(variant)) {
        e = x3.la.plain(x3.lp, s, true);
        if (e != hipSuccess) return HLA_ERR_DEVICE;
    }
    if (stage == 1 && p.nseg > 1) e = kern.summary(p, s);
    if (stage == 2 && p.nseg > 2 && !p.leaf_fold) e = kern.up_sweep(p, s);
    if (stage == 3) e = kern.forward(p, s);
    return e == hipSuccess ? HLA_OK : HLA_ERR_DEVICE;
}

hla_status hla_forward(const void *q, const void *k, const void *v, void *o, int B, int H, int n,
                       int d, int dv, int dtype, int variant, const float *gamma_host, int chunk,
                       int seg_chunks, const float *state_in, float *state_out, void *workspace,
                       size_t workspace_bytes, void *stream) {
    FwdKernels kern;
    FwdParams p;
    Hla3Pass x3;
    hla_status st = prepare_forward(q, k, v, o, B, H, n, d, dv, dtype, variant, gamma_host, chunk,
                                    seg_chunks, state_in, state_out, workspace, workspace_bytes,
                                    &kern, &p, &x3);
    if (st != HLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int stage = 1; stage <= 3; ++stage) {
        st = run_stage(stage, kern, p, variant, d, dv, x3, s);
        if (st != HLA_OK) return st;
    }
    return HLA_OK;
}

hla_status hla_forward_z(const void *q, const void *k, const void *v, void *o, void *z, int B,
                         int H, int n, int d, int dv, int dtype, int variant,
                         const float *gamma_host, int chunk, int seg_chunks,
                         const float *state_in, float *state_out, void *workspace,
                         size_t workspace_bytes, void *stream) {
    FwdKernels kern;
    FwdParams p;
    Hla3Pass x3;
    hla_status st = prepare_forward(q, k, v, o, B, H, n, d, dv, dtype, variant, gamma_host, chunk,
                                    seg_chunks, state_in, state_out, workspace, workspace_bytes,
                                    &kern, &p, &x3);
    if (st != HLA_OK) return st;
    if (variant != HLA_HLA2 && variant != HLA_HLA2_RATIO && variant != HLA_AHLA &&
        variant != HLA_AHLA_RATIO)
        return HLA_ERR_UNSUPPORTED;
    if (n > 0 && !z) return HLA_ERR_NULL;
    if (!kern.forward_z) return HLA_ERR_UNSUPPORTED;
    if (z && (z == q || z == k || z == v || z == o)) return HLA_ERR_ARG;
    p.z_out = z;
    kern.forward = kern.forward_z;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int stage = 1; stage <= 3; ++stage) {
        st = run_stage(stage, kern, p, variant, d, dv, x3, s);
        if (st != HLA_OK) return st;
    }
    return HLA_OK;
}

hla_status hla_forward_stage(int stage, const void *q, const void *k, const void *v, void *o,
                             int B, int H, int n, int d, int dv, int dtype, int variant,
                             const float *gamma_host, int chunk, int seg_chunks,
                             const float *state_in, float *state_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
    if (stage < 1 || stage > 3) return HLA_ERR_ARG;
    FwdKernels kern;
    FwdParams p;
    Hla3Pass x3;
    hla_status st = prepare_forward(q, k, v, o, B, H, n, d, dv, dtype, variant, gamma_host, chunk,
                                    seg_chunks, state_in, state_out, workspace, workspace_bytes,
                                    &kern, &p, &x3);
    if (st != HLA_OK) return st;
    return run_stage(stage, kern, p, variant, d, dv, x3, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ backward
//
// HLA-2 as two chained first-order linear attentions, with z_t = S^K_t q_t:
//   Z = LA_g(Q, K, K),   O = LA_{g^2}(Q, Z, V),
//   LA_g(A, B, C)_t = sum_{s<=t} g^(t-s) (a_t . b_s) c_s.
// The vector-Jacobian product of LA_g is three passes of the same form, two
// of them anti-causal (RLA: sum over s >= t, weight g^(s-t)):
//   dA = LA_g(dOut, C, B),  dB = RLA_g(C, dOut, A),  dC = RLA_g(B, A, dOut).
// Through O: dQ += LA_{g^2}(dO, V, Z), dZ = RLA_{g^2}(V, dO, Q),
//            dV = RLA_{g^2}(Z, Q, dO);
// through Z (K is both key and value there): dQ += LA_g(dZ, K, K),
//            dK = RLA_g(K, dZ, Q) + RLA_g(K, Q, dZ), the two slots in one
//            pass with one state (the kernels' SYM form).
// dZ and dV read one state (sum dO Q^T and its transpose) and share two
// inputs, so they run as one pass (the kernels' DUAL form): five passes in
// dependency order; Z and dZ live in the workspace.  The first and last
// passes share b = c = K and the decay g, so the segment states of the first
// are kept and reused by the last.
//
// AHLA is LA(Q, K, LA(Q, K, V)) without decay: Y = LA(Q, K, V), O = LA(Q, K, Y).
// Its gradient: dQ = LA(dO, Y, K) + LA(dY, V, K), dY = RLA(K, Q, dO),
// dK = RLA(Y, dO, Q) + RLA(V, dY, Q), dV = RLA(K, Q, dY); the pairs
// (dY, first dK term) and (dV, second dK term) each share one state and run
// as DUAL passes.

int hla_backward_default_seg_chunks(int B, int H, int n) {
    if (B < 1 || H < 1 || n < 1) return 1;
    const long nch = ceil_div(n, kLaChunk);
    // about 512 workgroups per pass, two per compute unit: the fused (SYM,
    // DUAL) and fp32 kernels hold two, the plain bf16 kernel three.  Measured
    // at B*H = 128, n = 4096 (bf16 backward / ratio backward, ms): 16 chunks
    // per segment 0.442 / 2.40, 11 chunks 0.450 / 2.72, 8 chunks 0.494 / 2.50
    long nseg = ceil_div(512, (long)B * H);
    long g = ceil_div(nch, nseg);
    if (g < 2) g = 2;
    if (g > nch) g = nch;
    return (int)g;
}

// The passes run in fp32 for the ratio forms (their q, k gradient is a small
// difference of large terms, which bf16 intermediates do not resolve) and
// whenever the decay gradient is asked for (dL/dg is a sum of position-
// weighted row terms that nearly cancel: with bf16 Z, dZ and gradients it is
// off by a few percent, with fp32 passes by about 1e-6 of itself).
static bool fp32_passes(int variant, bool with_dgamma) {
    return is_ratio(variant) || with_dgamma;
}
// tensors of [B][H][n][d] the backward keeps in its workspace: Z and dZ (Y
// and dY for AHLA); the ratio form adds dO / den, the rows (e, 0, ..., 0)
// and the unit rows (1, 0, ..., 0); fp32 passes on bf16 inputs run on
// widened copies of q, k, v, dO and fp32 gradients (seven more)
static int own_tensors(int variant) {
    switch (variant) {
        case HLA_HLA2_RATIO: return 5;
        case HLA_AHLA_RATIO: return 7;    // AHLA adds Y1, dY1
        case HLA_HLA3: return 4;
        case HLA_HLA3_RATIO: return 12;
        default: return 2;
    }
}
static int backward_tensors(int variant, int dtype, bool with_dgamma) {
    const int own = own_tensors(variant);
    return (fp32_passes(variant, with_dgamma) && dtype == HLA_BF16) ? own + 7 : own;
}
static size_t backward_elem_bytes(int variant, int dtype, bool with_dgamma) {
    return (fp32_passes(variant, with_dgamma) || dtype == HLA_F32) ? 4 : 2;
}
static bool has_backward(int variant) { return valid_variant(variant); }
// fp64 partial sums of the decay gradient, after the tensors (HLA-2 forms)
static size_t decay_grad_bytes(int variant, int B, int H) {
    const bool hla2 = variant == HLA_HLA2 || variant == HLA_HLA2_RATIO;
    return hla2 ? (size_t)B * H * kDecayGradBlocks * sizeof(double) : 0;
}

size_t hla_backward_workspace_bytes(int variant, int B, int H, int n, int d, int dv, int dtype,
                                    int seg_chunks, int with_dgamma) {
    if (!has_backward(variant) || B < 1 ||
        H < 1 || n < 1 || d < 1 || dv < 1 || seg_chunks < 0 ||
        (dtype != HLA_F32 && dtype != HLA_BF16))
        return 0;
    const bool dg = with_dgamma != 0;
    const int g = seg_chunks > 0 ? seg_chunks : hla_backward_default_seg_chunks(B, H, n);
    const long nseg = num_segments(n, kLaChunk, g);
    const size_t esz = backward_elem_bytes(variant, dtype, dg);
    const size_t sums = (size_t)B * H * (size_t)(nseg - 1) * d * d * sizeof(float);
    return 2 * sums + (size_t)backward_tensors(variant, dtype, dg) * B * H * n * d * esz +
           decay_grad_bytes(variant, B, H);
}


static hla_status backward_impl(const void *q, const void *k, const void *v, const void *z,
                                const void *dout, void *dq, void *dk, void *dv_out, int B, int H,
                                int n, int d, int dv, int dtype, int variant,
                                const float *gamma_host, float *dgamma, int seg_chunks,
                                void *workspace, size_t workspace_bytes, void *stream) {
    hla_status st = check_common(B, H, d, dv, dtype, variant, gamma_host);
    if (st != HLA_OK) return st;
    if (n < 0) return HLA_ERR_SHAPE;
    if (seg_chunks < 0) return HLA_ERR_ARG;
    if (!has_backward(variant) || d != dv) return HLA_ERR_UNSUPPORTED;
    // the decay gradient's identity is written for the HLA-2 chain
    if (dgamma && (is_ahla(variant) || is_hla3(variant))) return HLA_ERR_UNSUPPORTED;
    const bool dg = dgamma != nullptr;
    const bool fp32run = fp32_passes(variant, dg);
    const int run_dtype = fp32run ? HLA_F32 : dtype;
    BwdCtx c;
    c.p3_cube = is_hla3(variant);
    if (!lookup_la(run_dtype, d, &c.la)) return HLA_ERR_UNSUPPORTED;
    if (n == 0) {
        if (!dgamma) return HLA_OK;
        // no rows: dgamma = 0 (the second step of the decay gradient alone)
        DecayGradParams p;
        memset(&p, 0, sizeof(p));
        p.dgamma = dgamma;
        p.BH = B * H;
        p.H = H;
        for (int h = 0; h < kMaxDecayHeads; ++h) p.gamma[h] = 1.f;
        return c.la.decay_grad(p, static_cast<hipStream_t>(stream)) == hipSuccess
                   ? HLA_OK : HLA_ERR_DEVICE;
    }
    if (!q || !k || !v || !dout || !dq || !dk || !dv_out) return HLA_ERR_NULL;
    const int g = seg_chunks > 0 ? seg_chunks : hla_backward_default_seg_chunks(B, H, n);
    if ((long)kLaChunk * g > INT32_MAX / 2) return HLA_ERR_UNSUPPORTED;
    const long nseg = num_segments(n, kLaChunk, g);
    if (nseg * B * H > INT32_MAX / 2) return HLA_ERR_UNSUPPORTED;
    if ((long)B * H * n / 4 > INT32_MAX / 2) return HLA_ERR_UNSUPPORTED;   // row-wise grid
    const size_t need = hla_backward_workspace_bytes(variant, B, H, n, d, dv, dtype, g, dg);
    if (!workspace) return HLA_ERR_NULL;
    if (workspace_bytes < need) return HLA_ERR_WORKSPACE;

    // workspace: the K K^T segment states (kept from the first pass to the
    // last), the other passes' segment states, then [B*H*n*d] tensors
    c.ws = static_cast<char *>(workspace);
    c.sums_bytes = (size_t)B * H * (size_t)(nseg - 1) * d * d * sizeof(float);
    c.tensor_bytes = (size_t)B * H * n * d * backward_elem_bytes(variant, dtype, dg);
    c.sums_kk = reinterpret_cast<float *>(c.ws);
    c.sums = reinterpret_cast<float *>(c.ws + c.sums_bytes);
    c.rows = (long)B * H * n;
    c.s = static_cast<hipStream_t>(stream);
    memset(&c.p1, 0, sizeof(c.p1));   // decay g
    c.p1.BH = B * H;
    c.p1.H = H;
    c.p1.n = n;
    c.p1.seg_len = kLaChunk * g;
    c.p1.nseg = (int)nseg;
    fill_gamma(c.p1.gamma, gamma_host, H);
    c.p2 = c.p1;                      // decay g^2 (third order: g^3)
    for (int h = 0; h < kMaxDecayHeads; ++h)
        c.p2.gamma[h] = c.p1.gamma[h] * c.p1.gamma[h] * (c.p3_cube ? c.p1.gamma[h] : 1.f);

    Grads io{q, k, v, dout, dq, dk, dv_out, z};
    void *partial = c.tensor(backward_tensors(variant, dtype, dg));
    // fp32 passes on bf16 inputs read and write fp32 copies (after the
    // variant's own tensors in the workspace)
    Grads run = io;
    const int own = own_tensors(variant);
    const long count = c.rows * d;
    const bool widen = fp32run && dtype == HLA_BF16;
    if (widen) {
        const void *src[4] = {q, k, v, dout};
        const void **dst_in[4] = {&run.q, &run.k, &run.v, &run.dout};
        for (int i = 0; i < 4; ++i) {
            *dst_in[i] = c.tensor(own + i);
            if (launch_convert(src[i], c.tensor(own + i), count, true, c.s) != hipSuccess)
                return HLA_ERR_DEVICE;
        }
        run.dq = c.tensor(own + 4);
        run.dk = c.tensor(own + 5);
        run.dv = c.tensor(own + 6);
    }
    switch (variant) {
        case HLA_HLA2: st = backward_hla2(c, run); break;
        case HLA_AHLA: st = backward_ahla(c, run); break;
        case HLA_HLA2_RATIO: st = backward_hla2_ratio(c, run); break;
        case HLA_AHLA_RATIO: st = backward_ahla_ratio(c, run); break;
        default: st = backward_hla3(c, run, variant == HLA_HLA3_RATIO); break;
    }
    if (st == HLA_OK && dgamma) st = decay_gradient(c, run, H, n, d, dgamma, partial);
    if (st != HLA_OK || !widen) return st;
    void *dst[3] = {dq, dk, dv_out};
    const void *src[3] = {run.dq, run.dk, run.dv};
    for (int i = 0; i < 3; ++i)
        if (launch_convert(src[i], dst[i], count, false, c.s) != hipSuccess) return HLA_ERR_DEVICE;
    return HLA_OK;
}

hla_status hla_backward(const void *q, const void *k, const void *v, const void *dout, void *dq,
                        void *dk, void *dv_out, int B, int H, int n, int d, int dv, int dtype,
                        int variant, const float *gamma_host, float *dgamma, int seg_chunks,
                        void *workspace, size_t workspace_bytes, void *stream) {
    return backward_impl(q, k, v, nullptr, dout, dq, dk, dv_out, B, H, n, d, dv, dtype, variant,
                         gamma_host, dgamma, seg_chunks, workspace, workspace_bytes, stream);
}

hla_status hla_backward_z(const void *q, const void *k, const void *v, const void *z,
                          const void *dout, void *dq, void *dk, void *dv_out, int B, int H, int n,
                          int d, int dv, int dtype, int variant, const float *gamma_host,
                          int seg_chunks, void *workspace, size_t workspace_bytes, void *stream) {
    hla_status st = check_common(B, H, d, dv, dtype, variant, gamma_host);
    if (st != HLA_OK) return st;
    if (variant != HLA_HLA2 && variant != HLA_AHLA) return HLA_ERR_UNSUPPORTED;
    if (n > 0 && !z) return HLA_ERR_NULL;
    if (z && (z == dq || z == dk || z == dv_out)) return HLA_ERR_ARG;
    return backward_impl(q, k, v, z, dout, dq, dk, dv_out, B, H, n, d, dv, dtype, variant,
                         gamma_host, nullptr, seg_chunks, workspace, workspace_bytes, stream);
}

hla_status hla_step(const void *q, const void *k, const void *v, void *o, int B, int H, int d,
                    int dv, int dtype, int variant, const float *gamma_host, float *state,
                    void *stream) {
    hla_status st = check_common(B, H, d, dv, dtype, variant, gamma_host);
    if (st != HLA_OK) return st;
    if (!q || !k || !v || !o || !state) return HLA_ERR_NULL;
    StepLaunch fn;
    const int mode = is_hla3(variant) ? kStepHla3 : is_ahla(variant) ? kStepAhla : kStepHla2;
    if (!lookup_step(dtype, mode, d, dv, &fn)) return HLA_ERR_UNSUPPORTED;
    StepParams p;
    memset(&p, 0, sizeof(p));
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.state = state;
    p.BH = B * H;
    p.H = H;
    p.ratio = is_ratio(variant) ? 1 : 0;
    fill_gamma(p.gamma, gamma_host, H);
    if (fn(p, static_cast<hipStream_t>(stream)) != hipSuccess) return HLA_ERR_DEVICE;
    return HLA_OK;
}

const char *hla_status_str(int status) {
    switch (status) {
        case HLA_OK: return "ok";
        case HLA_ERR_NULL: return "a required pointer is NULL";
        case HLA_ERR_SHAPE: return "bad shape (B, H, d, dv must be >= 1 and n >= 0)";
        case HLA_ERR_UNSUPPORTED: return "no kernel for this dtype / d / dv / chunk / variant";
        case HLA_ERR_WORKSPACE: return "workspace smaller than hla_workspace_bytes()";
        case HLA_ERR_DEVICE: return "a HIP launch or runtime call failed";
        case HLA_ERR_ARG: return "bad argument value (enum, gamma outside (0, 1], negative chunk)";
        default: return "unknown status";
    }
}

}  // extern "C"

// Validation of hla_forward's arguments without a caller workspace: every
// check of prepare_forward except the workspace's own, and the workspace
// size the call needs.  No HIP call.
hla_status hla::forward_validate(const void *q, const void *k, const void *v, void *o, int B,
                                 int H, int n, int d, int dv, int dtype, int variant,
                                 const float *gamma_host, int chunk, int seg_chunks,
                                 const float *state_in, float *state_out, size_t *need) {
    FwdKernels kern;
    FwdParams p;
    Hla3Pass x3;
    // a stand-in address that passes the workspace checks; prepare_forward
    // only stores it, and it never reaches a kernel
    static char stand_in;
    hla_status st = prepare_forward(q, k, v, o, B, H, n, d, dv, dtype, variant, gamma_host, chunk,
                                    seg_chunks, state_in, state_out, &stand_in, SIZE_MAX, &kern,
                                    &p, &x3);
    if (st != HLA_OK) return st;
    const int g = effective_seg_chunks(variant, B, H, n, d, chunk, seg_chunks);
    *need = n > 0 ? hla_workspace_bytes(variant, B, H, n, d, dv, chunk, g) : 0;
    return HLA_OK;
}
