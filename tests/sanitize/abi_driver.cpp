// Host-side check of the C ABI's argument handling under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU: hla_api.cpp is linked against
// stand-ins for its kernel lookups whose "launches" only record their
// argument blocks.  Every call below either fails validation (its status is
// checked) or runs the whole host path -- workspace carving, pass lists,
// parameter blocks -- and every device pointer a launch receives is checked
// to lie inside the caller's buffers or the workspace it was given.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "hla.h"
#include "launch.h"

namespace {

struct Range {
    const char *lo, *hi;
};
std::vector<Range> g_ok;    // buffers a launch may point into
int g_launches = 0, g_bad = 0;

void allow(const void *p, size_t bytes) {
    g_ok.push_back({static_cast<const char *>(p), static_cast<const char *>(p) + bytes});
}
void check(const void *p, const char *what) {
    if (!p) return;
    const char *c = static_cast<const char *>(p);
    for (const Range &r : g_ok)
        if (c >= r.lo && c < r.hi) return;
    std::fprintf(stderr, "pointer %s = %p outside every buffer\n", what, p);
    ++g_bad;
}

hipError_t fwd_launch(const hla::FwdParams &p, hipStream_t) {
    ++g_launches;
    check(p.q, "q"); check(p.k, "k"); check(p.v, "v"); check(p.o, "o");
    check(p.ws, "ws"); check(p.state_in, "state_in"); check(p.state_out, "state_out");
    return hipSuccess;
}
hipError_t step_launch(const hla::StepParams &p, hipStream_t) {
    ++g_launches;
    check(p.q, "q"); check(p.state, "state");
    return hipSuccess;
}
hipError_t la_launch(const hla::LaParams &p, hipStream_t, bool) {
    ++g_launches;
    check(p.a, "a"); check(p.b, "b"); check(p.c, "c"); check(p.add, "add"); check(p.out, "out");
    check(p.a2, "a2"); check(p.out2, "out2"); check(p.add2, "add2"); check(p.sums, "sums");
    check(p.state_in, "state_in"); check(p.state_out, "state_out");
    check(p.state_out2, "state_out2");
    return hipSuccess;
}
hipError_t unit_launch(void *out, long, hipStream_t) { ++g_launches; check(out, "unit"); return hipSuccess; }
hipError_t prep_launch(const hla::RatioPrepParams &p, hipStream_t) {
    ++g_launches;
    check(p.q, "q"); check(p.u, "u"); check(p.num, "num"); check(p.dout, "dout");
    check(p.g, "g"); check(p.e1, "e1"); check(p.dq, "dq");
    return hipSuccess;
}
hipError_t dg_launch(const hla::DecayGradParams &p, hipStream_t) {
    ++g_launches;
    check(p.q, "q"); check(p.z, "z"); check(p.dz, "dz"); check(p.partial, "partial");
    check(p.dgamma, "dgamma");
    return hipSuccess;
}

}  // namespace

namespace hla {
bool lookup_forward(int dtype, bool, int d, int dv, int chunk, bool, FwdKernels *out) {
    if (d != dv || (chunk != 16 && chunk != 32 && chunk != 64)) return false;
    if (d != 16 && d != 32 && d != 64 && !(d == 128 && dtype == 1)) return false;
    *out = {fwd_launch, fwd_launch, fwd_launch};
    return true;
}
bool lookup_step(int, int, int d, int dv, StepLaunch *out) {
    if (d != dv) return false;
    *out = step_launch;
    return true;
}
bool lookup_la(int, int d, LaLaunches *out) {
    if (d != 16 && d != 32 && d != 64 && d != 128) return false;
    out->plain = out->sym = out->dual = la_launch;
    out->unit_column = unit_launch;
    out->ratio_prep = prep_launch;
    out->decay_grad = dg_launch;
    return true;
}
hipError_t launch_convert(const void *src, void *dst, long, bool, hipStream_t) {
    ++g_launches;
    check(src, "convert src"); check(dst, "convert dst");
    return hipSuccess;
}
hipError_t launch_divide_rows(const float *num, const float *den, void *out, long, int, bool,
                              hipStream_t) {
    ++g_launches;
    check(num, "num"); check(den, "den"); check(out, "out");
    return hipSuccess;
}
hipError_t launch_copy_or_zero(const float *src, float *dst, size_t, hipStream_t) {
    ++g_launches;
    check(src, "copy src"); check(dst, "copy dst");
    return hipSuccess;
}
}  // namespace hla

static int g_fail = 0;
#define EXPECT(cond)                                                                  \
    do {                                                                              \
        if (!(cond)) {                                                                \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                                 \
        }                                                                             \
    } while (0)

int main() {
    const int variants[] = {HLA_HLA2, HLA_HLA2_RATIO, HLA_AHLA, HLA_AHLA_RATIO, HLA_HLA3,
                            HLA_HLA3_RATIO};
    std::vector<float> gam(8, 0.9f), bad(8, 1.5f);
    // host stand-ins for device buffers, sized exactly as the header requires
    for (int dtype : {HLA_F32, HLA_BF16}) {
        for (int variant : variants) {
            for (int d : {16, 64, 128}) {
                for (int n : {0, 1, 77, 300}) {
                    for (int decay : {0, 1}) {
                        const int B = 2, H = 4, chunk = 32, seg = 2;
                        const size_t esz = dtype == HLA_BF16 ? 2 : 4;
                        const size_t tensor = (size_t)B * H * (n > 0 ? n : 1) * d * esz;
                        std::vector<char> q(tensor), k(tensor), v(tensor), o(tensor), dout(tensor),
                            dq(tensor), dk(tensor), dv(tensor);
                        const size_t sf = hla_state_floats(variant, d, d);
                        std::vector<float> si(B * H * sf), so(B * H * sf), dg(H);
                        const size_t need = hla_workspace_bytes(variant, B, H, n, d, d, chunk, seg);
                        std::vector<char> ws(need > 0 ? need : 1);
                        g_ok.clear();
                        for (auto *b : {&q, &k, &v, &o, &dout, &dq, &dk, &dv, &ws}) allow(b->data(), b->size());
                        allow(si.data(), si.size() * 4);
                        allow(so.data(), so.size() * 4);
                        allow(dg.data(), dg.size() * 4);
                        const float *g = decay ? gam.data() : nullptr;
                        hla_status st = hla_forward(q.data(), k.data(), v.data(), o.data(), B, H, n, d, d,
                                                    dtype, variant, g, chunk, seg, si.data(), so.data(),
                                                    ws.data(), need, nullptr);
                        const bool f32_128 = dtype == HLA_F32 && d == 128;
                        EXPECT(st == (f32_128 ? HLA_ERR_UNSUPPORTED : HLA_OK));
                        if (need > 0)
                            EXPECT(hla_forward(q.data(), k.data(), v.data(), o.data(), B, H, n, d, d,
                                               dtype, variant, g, chunk, seg, nullptr, nullptr,
                                               ws.data(), need - 1, nullptr) ==
                                   (f32_128 ? HLA_ERR_UNSUPPORTED : HLA_ERR_WORKSPACE));
                        for (int stage = 1; stage <= 3; ++stage)
                            hla_forward_stage(stage, q.data(), k.data(), v.data(), o.data(), B, H, n, d,
                                              d, dtype, variant, g, chunk, seg, nullptr, so.data(),
                                              ws.data(), need, nullptr);
                        EXPECT(hla_forward(q.data(), k.data(), v.data(), o.data(), B, H, n, d, d, dtype,
                                           variant, bad.data(), chunk, seg, nullptr, nullptr, ws.data(),
                                           need, nullptr) == HLA_ERR_ARG);
                        st = hla_step(q.data(), k.data(), v.data(), o.data(), B, H, d, d, dtype, variant,
                                      g, so.data(), nullptr);
                        EXPECT(st == HLA_OK);
                        // backward
                        const int with_dg = decay && (variant == HLA_HLA2 || variant == HLA_HLA2_RATIO);
                        const size_t bneed = hla_backward_workspace_bytes(variant, B, H, n, d, d, dtype,
                                                                          0, with_dg);
                        std::vector<char> bws(bneed > 0 ? bneed : 1);
                        allow(bws.data(), bws.size());
                        st = hla_backward(q.data(), k.data(), v.data(), dout.data(), dq.data(), dk.data(),
                                          dv.data(), B, H, n, d, d, dtype, variant, g,
                                          with_dg ? dg.data() : nullptr, 0, bws.data(), bneed, nullptr);
                        EXPECT(st == HLA_OK);
                        if (bneed > 0)
                            EXPECT(hla_backward(q.data(), k.data(), v.data(), dout.data(), dq.data(),
                                                dk.data(), dv.data(), B, H, n, d, d, dtype, variant, g,
                                                with_dg ? dg.data() : nullptr, 0, bws.data(), bneed - 1,
                                                nullptr) == (n == 0 ? HLA_OK : HLA_ERR_WORKSPACE));
                    }
                }
            }
        }
    }
    // argument errors, each before anything else happens
    float dummy[64];
    EXPECT(hla_forward(dummy, dummy, dummy, dummy, 0, 1, 8, 16, 16, 0, 0, nullptr, 16, 0, nullptr,
                       nullptr, nullptr, 0, nullptr) == HLA_ERR_SHAPE);
    EXPECT(hla_forward(nullptr, dummy, dummy, dummy, 1, 1, 8, 16, 16, 0, 0, nullptr, 16, 0,
                       nullptr, nullptr, nullptr, 0, nullptr) == HLA_ERR_NULL);
    EXPECT(hla_forward(dummy, dummy, dummy, dummy, 1, 1, 8, 16, 16, 0, 9, nullptr, 16, 0, nullptr,
                       nullptr, nullptr, 0, nullptr) == HLA_ERR_ARG);
    EXPECT(hla_workspace_bytes(9, 1, 1, 8, 16, 16, 16, 0) == 0);
    EXPECT(hla_state_floats(-1, 16, 16) == 0);
    EXPECT(hla_backward_workspace_bytes(2, 1, 1, 8, 16, 16, 7, 0, 0) == 0);
    for (int c = -1; c < 9; ++c) EXPECT(hla_status_str(c) != nullptr);
    std::printf("launches %d, pointers outside %d, failed expectations %d\n", g_launches, g_bad,
                g_fail);
    return (g_bad || g_fail) ? 1 : 0;
}
