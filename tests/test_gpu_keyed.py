"""The forward's first chained pass kept for the backward: hla_forward_z
writes the keyed queries z_t = S^K_t q_t of HLA-2 (S^K_t = sum_{s<=t}
g^(t-s) k_s k_s^T; "1. HLA de Segundo Orden" of "Resumen Tecnico: Atencion
Lineal de Orden Superior (HLA)", gist.science/es/paper/2510.27258) or the
rows y_t = P_t^T q_t of AHLA ("2. ... (AHLA)"), and hla_backward_z takes
them instead of recomputing Z = LA_g(Q, K, K) or Y = LA_g(Q, K, V).

Checked against the oracle: z element by element against the fp64
recurrences Z = LA_g(Q, K, K) and Y = LA_g(Q, K, V) of oracle/streaming_grad.py, the output bit for
bit against hla_forward's, and the gradients against the oracle's chain rule
(oracle/backward.py, oracle/streaming_grad.py) at the stated bar (1e-2
relative L2 for bf16, 1e-5 for fp32).  The cases cover every form of the
stage-3 kernel that writes z: the pipelined HLA-2 one (bf16, one wave per
row tile), the plain HLA-2 and AHLA ones with and without a decay, two column groups over a
swizzled (d = 64, chunk 32) and a padded (d = 128) tile, scans that fold
leaves (at most four segments) and scans with an up-sweep, ragged tails.
"""
import numpy as np
import pytest

from oracle import backward as BW
from oracle import streaming_grad as SG
from causal_streaming_scans_amd import inputs as I
from hla_testlib import TOL, from_dev, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, variant, d, n, H, decay, chunk, seg_chunks
    ("f32", "hla2", 16, 200, 2, False, 32, 2),
    ("f32", "hla2", 32, 130, 1, True, 16, 3),
    ("f32", "hla2_ratio", 64, 257, 2, False, 32, 1),
    ("bf16", "hla2", 16, 333, 2, True, 16, 4),
    ("bf16", "hla2", 32, 300, 2, False, 32, 2),
    ("bf16", "hla2", 64, 450, 3, False, 64, 2),        # pipelined, four segments
    ("bf16", "hla2_ratio", 64, 1000, 2, False, 64, 2),  # pipelined, eight segments (up-sweep)
    ("bf16", "hla2", 64, 700, 2, True, 64, 2),          # plain, decay
    ("bf16", "hla2", 64, 2100, 1, False, 64, 4),        # nine segments
    ("bf16", "hla2", 64, 200, 2, False, 32, 2),         # two column groups, swizzled tile
    ("bf16", "hla2", 128, 300, 2, True, 64, 1),         # two column groups, padded tile
    ("bf16", "hla2", 128, 200, 1, False, 32, 2),
    ("f32", "ahla", 32, 200, 1, False, 32, 2),
    ("bf16", "ahla", 64, 450, 2, False, 64, 2),
    ("bf16", "ahla", 64, 300, 2, True, 64, 2),
    ("bf16", "ahla_ratio", 64, 300, 2, False, 64, 1),
    ("bf16", "ahla", 64, 200, 2, False, 32, 2),         # two column groups, swizzled tile
    ("bf16", "ahla", 128, 200, 1, True, 64, 1),         # two column groups, padded tile
]


def _gammas(BH, H, gamma):
    return np.array([1.0 if gamma is None else float(gamma[bh % H]) for bh in range(BH)])


def _forward_pair(x, variant, B, H, dtype, chunk, seg, gamma):
    import torch
    import causal_streaming_scans_amd as hla
    n, d = x["q"].shape[1], x["q"].shape[2]
    shp = (B, H, n, d)
    q, k, v = (to_dev(x[key], dtype, shp) for key in ("q", "k", "v"))
    o_ref = hla.hla_forward(q, k, v, variant=variant, gamma=gamma, chunk=chunk, seg_chunks=seg)
    o, z = hla.hla_forward_z(q, k, v, variant=variant, gamma=gamma, chunk=chunk, seg_chunks=seg)
    torch.cuda.synchronize()
    return (q, k, v), o_ref, o, z


@pytest.mark.parametrize("dtype,variant,d,n,H,decay,chunk,seg", CASES)
def test_keyed_queries_and_backward(dtype, variant, d, n, H, decay, chunk, seg):
    import torch
    import causal_streaming_scans_amd as hla
    say(f"[keyed] {dtype} {variant} d {d} n {n} H {H} decay {decay} chunk {chunk} seg {seg}")
    B = 1
    dist = "uniform_pos" if variant.endswith("ratio") else (
        "normal_scaled" if dtype == "f32" else "l2norm")
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist=dist, seed=900 + d + n, decay=decay)
    gamma = x["gamma"]
    (q, k, v), o_ref, o, z = _forward_pair(x, variant, B, H, dtype, chunk, seg, gamma)
    assert torch.equal(o, o_ref)
    ahla = variant.startswith("ahla")
    # HLA-2: Z = LA_g(Q, K, K); AHLA: Y = LA_g(Q, K, V)
    want_z = SG.causal_la(x["q"].astype(np.float64), x["k"].astype(np.float64),
                          x["v" if ahla else "k"].astype(np.float64), _gammas(B * H, H, gamma))
    ez = rel_l2(from_dev(z).reshape(B * H, n, d), want_z)
    say(f"   z rel_l2 {ez:.3e}")
    assert ez < TOL[dtype]
    if variant not in ("hla2", "ahla"):
        return
    do = I.make_upstream_grad(B * H, n, d, dtype, seed=950 + n)
    dot = to_dev(do, dtype, (B, H, n, d))
    with_z = hla.hla_backward(q, k, v, dot, variant=variant, gamma=gamma, z=z)
    plain = hla.hla_backward(q, k, v, dot, variant=variant, gamma=gamma)
    torch.cuda.synchronize()
    if ahla:
        want = BW.ahla_vjp_batched(x["q"], x["k"], x["v"], do, H=H, gamma=gamma)
    else:
        want = BW.hla2_vjp_batched(x["q"], x["k"], x["v"], do, H, gamma)
    for name, g, p, w in zip(("dq", "dk", "dv"), with_z, plain, want):
        g = from_dev(g).reshape(B * H, n, d)
        e, ep = rel_l2(g, w), rel_l2(g, from_dev(p).reshape(B * H, n, d))
        say(f"   {name}: rel_l2 {e:.3e} (vs recomputed Z {ep:.3e})")
        assert e < TOL[dtype], (name, e)


def test_keyed_queries_ratio_n4096_sampled_heads():
    """The ratio workload B=8 H=16 n=4096 d=dv=64 bf16 in the default launch
    configuration (pipelined stage 3, four segments): o unchanged bit for
    bit, z of the first and last head against the oracle."""
    import torch
    import causal_streaming_scans_amd as hla
    w = I.WORKLOADS["ratio_n4096"]
    say(f"[keyed] workload {w.name}")
    x = I.workload_inputs("ratio_n4096")
    shp = (w.B, w.H, w.n, w.d)
    q, k, v = (to_dev(x[key], w.dtype, shp) for key in ("q", "k", "v"))
    o_ref = hla.hla_forward(q, k, v, variant=w.variant, chunk=w.chunk)
    o, z = hla.hla_forward_z(q, k, v, variant=w.variant, chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    heads = [0, w.B * w.H - 1]
    zf = from_dev(z).reshape(w.B * w.H, w.n, w.d)
    want = SG.causal_la(x["q"][heads].astype(np.float64), x["k"][heads].astype(np.float64),
                        x["k"][heads].astype(np.float64), np.ones(len(heads)))
    e = rel_l2(zf[heads], want)
    say(f"   z heads 0, 127: rel_l2 {e:.3e}")
    assert e < TOL[w.dtype]


def test_backward_z_decay_n16384_whole_heads():
    """The decay workload B=2 H=16 n=16384 d=dv=128 bf16 at full size: z and
    the gradients of two whole heads against the oracle's linear-time
    recurrences, and every head's gradients against the backward that
    recomputes Z."""
    import torch
    import causal_streaming_scans_amd as hla
    w = I.WORKLOADS["decay_n16384"]
    say(f"[keyed] workload {w.name}")
    x = I.workload_inputs("decay_n16384")
    BH = w.B * w.H
    shp = (w.B, w.H, w.n, w.d)
    q, k, v = (to_dev(x[key], w.dtype, shp) for key in ("q", "k", "v"))
    gamma = x["gamma"]
    o_ref = hla.hla_forward(q, k, v, variant=w.variant, gamma=gamma, chunk=w.chunk)
    o, z = hla.hla_forward_z(q, k, v, variant=w.variant, gamma=gamma, chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    heads = [3, BH - 1]
    g = _gammas(BH, w.H, gamma)[heads]
    xs = {key: x[key][heads].astype(np.float64) for key in ("q", "k", "v")}
    e = rel_l2(from_dev(z).reshape(BH, w.n, w.d)[heads], SG.causal_la(xs["q"], xs["k"], xs["k"], g))
    say(f"   z heads 3, 31: rel_l2 {e:.3e}")
    assert e < TOL[w.dtype]
    do = I.make_upstream_grad(BH, w.n, w.dv, w.dtype, seed=w.seed + 100)
    dot = to_dev(do, w.dtype, shp)
    with_z = hla.hla_backward(q, k, v, dot, gamma=gamma, z=z)
    plain = hla.hla_backward(q, k, v, dot, gamma=gamma)
    torch.cuda.synchronize()
    want = SG.hla2_vjp_streaming(xs["q"], xs["k"], xs["v"], do[heads],
                                 gamma=[gamma[bh % w.H] for bh in heads], H=len(heads))
    for name, gz, gp, wt in zip(("dq", "dk", "dv"), with_z, plain, want):
        gz = from_dev(gz).reshape(BH, w.n, w.d)
        e, ep = rel_l2(gz[heads], wt), rel_l2(gz, from_dev(gp).reshape(BH, w.n, w.d))
        say(f"   {name}: heads 3, 31 rel_l2 {e:.3e}; all heads vs recomputed Z {ep:.3e}")
        assert e < TOL[w.dtype] and ep < TOL[w.dtype], (name, e, ep)


def test_backward_z_ahla_n65536():
    """The AHLA workload B=1 H=32 n=65536 d=dv=64 bf16 in the default launch
    configuration (sixteen segments, a scan with an up-sweep): y of two whole
    heads against the oracle's recurrence Y = LA(Q, K, V), and every head's
    gradients against the backward that recomputes Y."""
    import torch
    import causal_streaming_scans_amd as hla
    w = I.WORKLOADS["ahla_n65536"]
    say(f"[keyed] workload {w.name}")
    x = I.workload_inputs("ahla_n65536", decode_tokens=0)
    BH = w.B * w.H
    shp = (w.B, w.H, w.n, w.d)
    q, k, v = (to_dev(x[key], w.dtype, shp) for key in ("q", "k", "v"))
    o_ref = hla.hla_forward(q, k, v, variant=w.variant, chunk=w.chunk)
    o, y = hla.hla_forward_z(q, k, v, variant=w.variant, chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    heads = [0, BH - 1]
    xs = {key: x[key][heads].astype(np.float64) for key in ("q", "k", "v")}
    e = rel_l2(from_dev(y).reshape(BH, w.n, w.dv)[heads],
               SG.causal_la(xs["q"], xs["k"], xs["v"], np.ones(len(heads))))
    say(f"   y heads 0, 31: rel_l2 {e:.3e}")
    assert e < TOL[w.dtype]
    do = I.make_upstream_grad(BH, w.n, w.dv, w.dtype, seed=w.seed + 100)
    dot = to_dev(do, w.dtype, shp)
    with_y = hla.hla_backward(q, k, v, dot, variant="ahla", z=y)
    plain = hla.hla_backward(q, k, v, dot, variant="ahla")
    torch.cuda.synchronize()
    for name, gy, gp in zip(("dq", "dk", "dv"), with_y, plain):
        ep = rel_l2(from_dev(gy), from_dev(gp))
        say(f"   {name}: all heads vs recomputed Y {ep:.3e}")
        assert ep < TOL[w.dtype], (name, ep)
