"""GPU parity of the third-order variant (hla_forward, variant "hla3") against
the fp64 oracle of oracle/third_order.py: o = tril(L L^T) L V, the strictly
causal reading of the product A A^T A of section "3. HLA de Tercer Orden"
("Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
gist.science/es/paper/2510.27258).  Relative L2: 1e-5 fp32, 1e-2 bf16."""
import pytest

from causal_streaming_scans_amd import inputs as I
from oracle import third_order as T3
from hla_testlib import TOL, from_dev, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, d, n, H, chunk, seg_chunks
    ("f32", 16, 200, 2, 32, 2),
    ("f32", 32, 130, 1, 16, 0),
    ("f32", 64, 257, 2, 64, 1),
    ("bf16", 16, 333, 2, 32, 3),
    ("bf16", 64, 65, 2, 64, 0),
    ("bf16", 64, 450, 3, 64, 2),
    ("bf16", 128, 300, 2, 32, 2),
]


def run(x, B, H, dtype, chunk, seg):
    import torch
    import causal_streaming_scans_amd as hla
    n, d = x["q"].shape[1], x["q"].shape[2]
    shp = (B, H, n, d)
    o = hla.hla_forward(to_dev(x["q"], dtype, shp), to_dev(x["k"], dtype, shp),
                        to_dev(x["v"], dtype, shp), variant="hla3", chunk=chunk, seg_chunks=seg)
    torch.cuda.synchronize()
    return from_dev(o).reshape(B * H, n, d)


@pytest.mark.parametrize("dtype,d,n,H,chunk,seg", CASES)
def test_hla3_small(dtype, d, n, H, chunk, seg):
    say(f"[third order] dtype {dtype} d {d} n {n} H {H} chunk {chunk} seg_chunks {seg}")
    B = 1
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="normal_scaled" if dtype == "f32" else "l2norm",
                      seed=990 + d + n)
    got = run(x, B, H, dtype, chunk, seg)
    want = T3.hla3_batched(x["q"], x["k"], x["v"])
    e = rel_l2(got, want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL[dtype]


def test_hla3_n2048_sampled_heads():
    """The HLA-2 workload's inputs (B=4 H=8 n=2048 d=dv=64 bf16) through the
    third-order variant in the default launch configuration; the oracle on
    the first and last head."""
    w = I.WORKLOADS["hla2_n2048"]
    say(f"[third order] inputs of {w.name}")
    x = I.workload_inputs("hla2_n2048")
    got = run(x, w.B, w.H, w.dtype, 64, 0)
    heads = [0, w.B * w.H - 1]
    want = T3.hla3_batched(x["q"], x["k"], x["v"], heads=heads)
    e = rel_l2(got[heads], want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL[w.dtype]


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("bf16", 64), ("bf16", 128)])
def test_hla3_resume_and_decode(dtype, d):
    """Streaming state of the third-order variant: a forward over the first
    n1 tokens with state_out, a forward over the next n2 tokens continuing
    from it (state_in), then decode steps (hla_step) continuing from that;
    every output against the oracle on the whole sequence."""
    import numpy as np
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n1, n2, T = 1, 3, 190, 150, 4
    n = n1 + n2 + T
    say(f"[third order] resume + decode dtype {dtype} d {d} n1 {n1} n2 {n2} steps {T}")
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="normal_scaled" if dtype == "f32" else "l2norm",
                      seed=1400 + d)
    want = T3.hla3_batched(x["q"], x["k"], x["v"])
    stf = hla.state_floats("hla3", d, d)
    st1 = torch.empty(B * H * stf, dtype=torch.float32, device="cuda")
    st2 = torch.empty_like(st1)

    def part(a, b):
        return tuple(to_dev(np.ascontiguousarray(x[key][:, a:b]), dtype, (B, H, b - a, d))
                     for key in ("q", "k", "v"))

    o1 = hla.hla_forward(*part(0, n1), variant="hla3", chunk=32, seg_chunks=2, state_out=st1)
    o2 = hla.hla_forward(*part(n1, n1 + n2), variant="hla3", chunk=64, seg_chunks=1, state_in=st1,
                         state_out=st2)
    outs = []
    for t in range(n1 + n2, n):
        qt, kt, vt = (to_dev(np.ascontiguousarray(x[key][:, t]), dtype, (B, H, d))
                      for key in ("q", "k", "v"))
        outs.append(hla.hla_step(qt, kt, vt, st2, variant="hla3"))
    torch.cuda.synchronize()
    got1 = from_dev(o1).reshape(B * H, n1, d)
    got2 = from_dev(o2).reshape(B * H, n2, d)
    got3 = np.stack([from_dev(o).reshape(B * H, d) for o in outs], axis=1)
    for label, g, w in (("first", got1, want[:, :n1]), ("resumed", got2, want[:, n1:n1 + n2]),
                        ("decode", got3, want[:, n1 + n2:])):
        e = rel_l2(g, w)
        say(f"  {label}: rel_l2 {e:.3e}")
        assert e < TOL[dtype], (label, e)


def test_hla3_stages_equal_whole():
    """hla_forward_stage 1, 2, 3 in order (stage 1 also runs the first-order
    pass into the workspace) give exactly hla_forward's output."""
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n, d, chunk, seg = 1, 2, 700, 64, 64, 2
    say(f"[third order] stages vs whole B={B} H={H} n={n} d={d}")
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist="l2norm", seed=1501)
    q, k, v = (to_dev(x[key], "bf16", (B, H, n, d)) for key in ("q", "k", "v"))
    whole = hla.hla_forward(q, k, v, variant="hla3", chunk=chunk, seg_chunks=seg)
    ws = torch.empty(hla.workspace_bytes("hla3", B, H, n, d, d, chunk, seg), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(whole)
    for stage in (1, 2, 3):
        hla.hla_forward_stage(stage, q, k, v, variant="hla3", chunk=chunk, seg_chunks=seg,
                              out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, whole)


# ------------------------------------------------- decay and the ratio form

CHAIN_CASES = [
    # dtype, variant, d, n, H, decay
    ("f32", "hla3", 16, 200, 2, True),
    ("f32", "hla3_ratio", 32, 130, 2, False),
    ("f32", "hla3_ratio", 64, 257, 2, True),
    ("bf16", "hla3", 64, 450, 3, True),
    ("bf16", "hla3", 128, 300, 2, True),
    ("bf16", "hla3_ratio", 64, 333, 2, False),
    ("bf16", "hla3_ratio", 64, 700, 2, True),
    ("bf16", "hla3_ratio", 128, 200, 2, True),
    ("bf16", "hla3", 32, 65, 2, True),
]


def run_chain(x, B, H, dtype, variant, gamma, state_in=None, state_out=None):
    import torch
    import causal_streaming_scans_amd as hla
    n, d = x["q"].shape[1], x["q"].shape[2]
    shp = (B, H, n, d)
    o = hla.hla_forward(*(to_dev(x[a], dtype, shp) for a in "qkv"), variant=variant, gamma=gamma,
                        state_in=state_in, state_out=state_out)
    torch.cuda.synchronize()
    return from_dev(o).reshape(B * H, n, d)


@pytest.mark.parametrize("dtype,variant,d,n,H,decay", CHAIN_CASES)
def test_hla3_decay_and_ratio(dtype, variant, d, n, H, decay):
    """Third order with per-head decays (every moment decays by g per token)
    and its ratio form, through the chained first-order passes."""
    say(f"[third order] {variant} dtype {dtype} d {d} n {n} H {H} decay {decay}")
    B = 2
    ratio = variant == "hla3_ratio"
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="uniform_pos" if ratio else "l2norm",
                      seed=1600 + d + n, decay=decay)
    got = run_chain(x, B, H, dtype, variant, x["gamma"])
    want = T3.hla3_batched(x["q"], x["k"], x["v"], H=H, gamma=x["gamma"], ratio=ratio)
    e = rel_l2(got, want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL[dtype]


@pytest.mark.parametrize("dtype,variant,d", [("f32", "hla3", 32), ("bf16", "hla3", 64),
                                             ("bf16", "hla3_ratio", 64), ("f32", "hla3_ratio", 16),
                                             ("bf16", "hla3", 128)])
def test_hla3_decay_resume_and_decode(dtype, variant, d):
    """With a decay: forward over n1 tokens with state_out, a resumed forward
    over n2 tokens, then decode steps, each against the oracle on the whole
    sequence (the state carries P, S and W for each chain)."""
    import numpy as np
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n1, n2, T = 1, 3, 190, 141, 4
    n = n1 + n2 + T
    ratio = variant == "hla3_ratio"
    say(f"[third order] resume + decode {variant} {dtype} d {d} n1 {n1} n2 {n2} steps {T}")
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="uniform_pos" if ratio else "l2norm",
                      seed=1700 + d, decay=True)
    g = x["gamma"]
    want = T3.hla3_batched(x["q"], x["k"], x["v"], H=H, gamma=g, ratio=ratio)
    stf = hla.state_floats(variant, d, d)
    st1 = torch.empty(B * H * stf, dtype=torch.float32, device="cuda")
    st2 = torch.empty_like(st1)

    def part(a, b):
        return {key: np.ascontiguousarray(x[key][:, a:b]) for key in ("q", "k", "v")}

    got1 = run_chain(part(0, n1), B, H, dtype, variant, g, state_out=st1)
    got2 = run_chain(part(n1, n1 + n2), B, H, dtype, variant, g, state_in=st1, state_out=st2)
    outs = []
    for t in range(n1 + n2, n):
        qt, kt, vt = (to_dev(np.ascontiguousarray(x[key][:, t]), dtype, (B, H, d))
                      for key in ("q", "k", "v"))
        outs.append(hla.hla_step(qt, kt, vt, st2, variant=variant, gamma=g))
    torch.cuda.synchronize()
    got3 = np.stack([from_dev(o).reshape(B * H, d) for o in outs], axis=1)
    for label, gg, w in (("first", got1, want[:, :n1]), ("resumed", got2, want[:, n1:n1 + n2]),
                         ("decode", got3, want[:, n1 + n2:])):
        e = rel_l2(gg, w)
        say(f"  {label}: rel_l2 {e:.3e}")
        assert e < TOL[dtype], (label, e)


def test_hla3_ratio_n2048_sampled_heads():
    """The ratio form with decays g_h ~ U[0.95, 0.999] at the HLA-2 workload's
    shape (B=4 H=8 n=2048 d=dv=64 bf16, q, k ~ U[0,1)/sqrt(d)); the oracle on
    the first and last head."""
    w = I.WORKLOADS["hla2_n2048"]
    say("[third order] ratio with decay, B=4 H=8 n=2048 d=64 bf16")
    x = I.make_inputs(w.B, w.H, w.n, w.d, w.dv, dtype="bf16", dist="uniform_pos", seed=1801,
                      decay=True)
    got = run_chain(x, w.B, w.H, "bf16", "hla3_ratio", x["gamma"])
    heads = [0, w.B * w.H - 1]
    want = T3.hla3_batched(x["q"], x["k"], x["v"], heads=heads, H=w.H, gamma=x["gamma"], ratio=True)
    e = rel_l2(got[heads], want)
    say(f"  rel_l2 {e:.3e}")
    assert e < TOL["bf16"]


# ------------------------------------------------------------------ backward

BWD_CASES = [
    # dtype, variant, d, n, H, decay, seg_chunks
    ("f32", "hla3", 16, 200, 2, False, 1),
    ("f32", "hla3", 32, 130, 2, True, 0),
    ("f32", "hla3_ratio", 32, 150, 2, True, 1),
    ("bf16", "hla3", 64, 450, 3, False, 2),
    ("bf16", "hla3", 64, 333, 2, True, 1),
    ("bf16", "hla3", 128, 300, 2, True, 1),
    ("bf16", "hla3_ratio", 64, 300, 2, False, 1),
    ("bf16", "hla3_ratio", 16, 257, 2, True, 0),
    ("bf16", "hla3", 16, 65, 2, True, 0),
]


@pytest.mark.parametrize("dtype,variant,d,n,H,decay,seg", BWD_CASES)
def test_hla3_backward(dtype, variant, d, n, H, decay, seg):
    """Gradients of the third-order operator (and its ratio form, with and
    without decays) against the oracle's chain rule through its matrix form."""
    import torch
    import causal_streaming_scans_amd as hla
    from oracle import third_order as T
    say(f"[third order backward] {variant} {dtype} d {d} n {n} H {H} decay {decay} seg {seg}")
    B = 1
    ratio = variant == "hla3_ratio"
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="uniform_pos" if ratio else "l2norm",
                      seed=1900 + d + n, decay=decay)
    do = I.make_upstream_grad(B * H, n, d, dtype, seed=1950 + n)
    shp = (B, H, n, d)
    got = hla.hla_backward(*(to_dev(x[a], dtype, shp) for a in "qkv"), to_dev(do, dtype, shp),
                           variant=variant, gamma=x["gamma"], seg_chunks=seg)
    torch.cuda.synchronize()
    want = T.hla3_vjp_batched(x["q"], x["k"], x["v"], do, H=H, gamma=x["gamma"], ratio=ratio)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        e = rel_l2(from_dev(g).reshape(w.shape), w)
        say(f"  {name}: rel_l2 {e:.3e}")
        assert e < TOL[dtype], (name, e)
