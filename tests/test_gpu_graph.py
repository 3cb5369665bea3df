"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must equal the eager result exactly (the kernels use
fixed-order reductions), with eager work and synchronisation between the
replays.  The library records no memset into a captured stream; these tests
hold it to that by checking each replay, not only the first."""
import numpy as np
import pytest

from causal_streaming_scans_amd import inputs as I
from hla_testlib import TOL, from_dev, oracle_forward, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


def _capture(fn, stream):
    import torch
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fn()                       # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("variant,decay", [("hla2_ratio", False), ("hla2", True), ("ahla", False)])
def test_forward_graph_replay(variant, decay):
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n, d, chunk, seg = 2, 3, 1000, 64, 64, 3      # 6 segments, ragged tail
    say(f"[graph] forward {variant} decay={decay} B={B} H={H} n={n} d={d}")
    dist = "uniform_pos" if variant.endswith("ratio") else "l2norm"
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist=dist, seed=901, decay=decay)
    q = to_dev(x["q"], "bf16", (B, H, n, d))
    k = to_dev(x["k"], "bf16", (B, H, n, d))
    v = to_dev(x["v"], "bf16", (B, H, n, d))
    eager = hla.hla_forward(q, k, v, variant=variant, gamma=x["gamma"], chunk=chunk,
                            seg_chunks=seg).clone()
    torch.cuda.synchronize()
    want = oracle_forward(x, variant, H, gamma=x["gamma"])
    assert rel_l2(from_dev(eager).reshape(want.shape), want) < TOL["bf16"]

    s = torch.cuda.Stream()
    out = torch.empty_like(eager)
    ws = torch.empty(max(1, hla.workspace_bytes(variant, B, H, n, d, d, chunk, seg)),
                     dtype=torch.uint8, device="cuda")
    plan = hla.ForwardPlan(q, k, v, variant=variant, gamma=x["gamma"], chunk=chunk,
                           seg_chunks=seg, out=out, workspace=ws, stream=s)
    g = _capture(plan.run, s)
    for r in range(3):
        out.fill_(float("nan"))            # eager work between replays
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager forward"


def test_step_graph_replay():
    import torch
    import causal_streaming_scans_amd as hla
    B, H, d, T = 1, 8, 64, 16
    say(f"[graph] decode AHLA B={B} H={H} d={d}, {T} steps per graph")
    x = I.make_inputs(B, H, T, d, d, dtype="bf16", dist="l2norm", seed=902)
    stf = hla.state_floats("ahla", d, d)
    state0 = torch.from_numpy(
        np.random.default_rng(3).standard_normal(B * H * stf).astype(np.float32) * 0.1).cuda()
    qs = [to_dev(x["q"][:, t], "bf16", (B, H, d)) for t in range(T)]
    ks = [to_dev(x["k"][:, t], "bf16", (B, H, d)) for t in range(T)]
    vs = [to_dev(x["v"][:, t], "bf16", (B, H, d)) for t in range(T)]

    st_e = state0.clone()
    outs_e = [hla.hla_step(qs[t], ks[t], vs[t], st_e, variant="ahla").clone() for t in range(T)]
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    state = state0.clone()
    outs = [torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(T)]
    plans = [hla.StepPlan(qs[t], ks[t], vs[t], state, variant="ahla", out=outs[t], stream=s)
             for t in range(T)]

    def run_all():
        for p in plans:
            p.run()

    g = _capture(run_all, s)
    for r in range(3):
        state.copy_(state0)                # eager work between replays
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, st_e), f"replay {r}: state differs from {T} eager steps"
        for t in range(T):
            assert torch.equal(outs[t], outs_e[t]), f"replay {r}: output of step {t} differs"


@pytest.mark.parametrize("variant,decay", [("hla2", True), ("hla2_ratio", False), ("ahla", False)])
def test_backward_graph_replay(variant, decay):
    """hla_backward captured once and replayed: every replay equals the eager
    gradients bit for bit, with the workspace and outputs overwritten between
    replays (the backward fills its unit rows with a kernel, not a memset)."""
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n, d, seg = 1, 3, 900, 64, 3           # 5 segments, ragged tail
    say(f"[graph] backward {variant} decay={decay} B={B} H={H} n={n} d={d}")
    dist = "uniform_pos" if variant.endswith("ratio") else "l2norm"
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist=dist, seed=903, decay=decay)
    q, k, v = (to_dev(x[key], "bf16", (B, H, n, d)) for key in ("q", "k", "v"))
    do = to_dev(I.make_upstream_grad(B * H, n, d, "bf16", seed=904), "bf16", (B, H, n, d))
    eager = [t.clone() for t in hla.hla_backward(q, k, v, do, variant=variant, gamma=x["gamma"],
                                                 seg_chunks=seg)]
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    grads = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(max(1, hla.backward_workspace_bytes(variant, B, H, n, d, d, "bf16", seg)),
                     dtype=torch.uint8, device="cuda")
    plan = hla.BackwardPlan(q, k, v, do, variant=variant, gamma=x["gamma"], seg_chunks=seg,
                            dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws, stream=s)
    g = _capture(plan.run, s)
    for r in range(3):
        for t in grads:
            t.fill_(float("nan"))          # eager work between replays
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv"), grads, eager):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager backward"
