"""Edge cases of the newer entry points on the GPU: sequences shorter than a
chunk, exactly one chunk and one token past it, with several batch entries
and heads, for every backward variant and for the third-order forward and
decode; each against the fp64 oracle."""
import numpy as np
import pytest

from causal_streaming_scans_amd import inputs as I
from oracle import backward as BW
from oracle import third_order as T3
from hla_testlib import TOL, from_dev, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu

NS = [1, 17, 64, 65]


@pytest.mark.parametrize("variant", ["hla2", "hla2_ratio", "ahla", "ahla_ratio"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_short_sequences(variant, dtype):
    import torch
    import causal_streaming_scans_amd as hla
    B, H, d = 2, 2, 32
    for n in NS:
        say(f"[edges] backward {variant} {dtype} B={B} H={H} n={n} d={d}")
        dist = "uniform_pos" if variant.endswith("ratio") else "l2norm"
        x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist=dist, seed=1600 + n,
                          decay=variant == "hla2")
        do = I.make_upstream_grad(B * H, n, d, dtype, seed=1700 + n)
        shp = (B, H, n, d)
        gamma = x["gamma"] if variant == "hla2" else None
        got = hla.hla_backward(*(to_dev(x[key], dtype, shp) for key in ("q", "k", "v")),
                               to_dev(do, dtype, shp), variant=variant, gamma=gamma)
        torch.cuda.synchronize()
        ratio = variant.endswith("ratio")
        if variant.startswith("hla2"):
            want = BW.hla2_vjp_batched(x["q"], x["k"], x["v"], do, H, gamma, ratio=ratio)
        else:
            want = BW.ahla_vjp_batched(x["q"], x["k"], x["v"], do, ratio=ratio)
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            g = from_dev(g).reshape(w.shape)
            if ratio and n == 1 and name != "dv":
                # one token: the ratio output is v itself, so the q and k
                # gradients vanish; compare to their natural scale instead
                # of to a zero reference
                scale = np.linalg.norm(do) * np.linalg.norm(x["v"]) / np.linalg.norm(
                    x["q"] if name == "dq" else x["k"])
                e = float(np.linalg.norm(g - w) / scale)
            else:
                e = rel_l2(g, w)
            assert e < TOL[dtype], (n, name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_third_order_short_sequences_and_decode(dtype):
    import torch
    import causal_streaming_scans_amd as hla
    B, H, d = 2, 2, 32
    for n in NS:
        say(f"[edges] third order {dtype} B={B} H={H} n={n} d={d}, then one decode step")
        x = I.make_inputs(B, H, n + 1, d, d, dtype=dtype, dist="l2norm", seed=1800 + n)
        want = T3.hla3_batched(x["q"], x["k"], x["v"])
        shp = (B, H, n, d)
        st = torch.empty(B * H * hla.state_floats("hla3", d, d), dtype=torch.float32, device="cuda")
        o = hla.hla_forward(*(to_dev(np.ascontiguousarray(x[key][:, :n]), dtype, shp)
                              for key in ("q", "k", "v")), variant="hla3", state_out=st)
        od = hla.hla_step(*(to_dev(np.ascontiguousarray(x[key][:, n]), dtype, (B, H, d))
                            for key in ("q", "k", "v")), st, variant="hla3")
        torch.cuda.synchronize()
        assert rel_l2(from_dev(o).reshape(B * H, n, d), want[:, :n]) < TOL[dtype], n
        assert rel_l2(from_dev(od).reshape(B * H, d), want[:, n]) < TOL[dtype], n


@pytest.mark.parametrize("variant", ["hla2_ratio", "ahla_ratio"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_denominator_rows(variant, dtype):
    """A ratio row whose denominator is exactly zero.  With q_t = 0 every
    score A[t, i] of row t vanishes, so num_t = den_t = 0 and the row is 0/0.
    The header promises IEEE behaviour (no epsilon): that row is NaN in every
    column, in the oracle as on the GPU, and every other row is finite and
    matches the oracle (the zero rows change nothing else: q_t enters the
    later rows only through the moments, and a zero q adds nothing there)."""
    B, H, n, d = 1, 2, 200, 32
    zero_rows = [0, 70, 199]
    say(f"[edges] zero denominator {variant} {dtype} n={n} rows {zero_rows}")
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="uniform_pos", seed=2100,
                      decay=variant == "hla2_ratio")
    x["q"][:, zero_rows, :] = 0.0
    gamma = x["gamma"]
    from hla_testlib import gpu_forward, oracle_forward
    got = gpu_forward(x, variant, B, H, dtype, 32, 2, gamma=gamma)
    with np.errstate(invalid="ignore", divide="ignore"):
        want = oracle_forward(x, variant, H, gamma=gamma)
    keep = np.setdiff1d(np.arange(n), zero_rows)
    assert np.isnan(want[:, zero_rows]).all()
    assert np.isnan(got[:, zero_rows]).all()
    assert np.isfinite(got[:, keep]).all()
    err = rel_l2(got[:, keep], want[:, keep])
    say(f"   other rows rel_l2 {err:.3e}")
    assert err < TOL[dtype]


def _poisoned(nbytes, fill):
    import torch
    words = max(1, -(-nbytes // 4))
    return torch.full((words,), fill, dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("variant", ["hla2_ratio", "ahla", "hla3"])
def test_forward_ignores_workspace_contents(variant):
    """The workspace's contents on entry are ignored (header): a workspace
    filled with NaN gives the same output and state, bit for bit, as a
    zeroed one, on a launch with many segments (every part of the scan's
    workspace is written before it is read)."""
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n, d, chunk, seg = 2, 2, 700, 64, 32, 2
    say(f"[edges] poisoned forward workspace {variant} n={n} seg={seg}")
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist="uniform_pos", seed=2200,
                      decay=variant.startswith("hla2"))
    shp = (B, H, n, d)
    q, k, v = (to_dev(x[a], "bf16", shp) for a in "qkv")
    need = hla.workspace_bytes(variant, B, H, n, d, d, chunk, seg)
    assert need > 0
    outs = []
    for fill in (0.0, float("nan")):
        ws = _poisoned(need, fill)
        st = torch.full((B * H * hla.state_floats(variant, d, d),), fill, device="cuda")
        o = hla.hla_forward(q, k, v, variant=variant, gamma=x["gamma"] if variant.startswith("hla2") else None,
                            chunk=chunk, seg_chunks=seg, state_out=st, workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.clone(), st.clone()))
    assert torch.isfinite(outs[1][0].float()).all()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("variant", ["hla2", "hla2_ratio", "ahla"])
def test_backward_ignores_workspace_contents(variant):
    """As for the forward: the backward's workspace may hold anything."""
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n, d, seg = 2, 2, 600, 32, 2
    say(f"[edges] poisoned backward workspace {variant} n={n} seg={seg}")
    dist = "uniform_pos" if variant.endswith("ratio") else "l2norm"
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist=dist, seed=2300,
                      decay=variant.startswith("hla2"))
    do = I.make_upstream_grad(B * H, n, d, "bf16", seed=2301)
    shp = (B, H, n, d)
    args = [to_dev(x[a], "bf16", shp) for a in "qkv"] + [to_dev(do, "bf16", shp)]
    need = hla.backward_workspace_bytes(variant, B, H, n, d, d, "bf16", seg)
    res = []
    for fill in (0.0, float("nan")):
        ws = _poisoned(need, fill)
        g = hla.hla_backward(*args, variant=variant, seg_chunks=seg, workspace=ws,
                             gamma=x["gamma"] if variant.startswith("hla2") else None)
        torch.cuda.synchronize()
        res.append([t.clone() for t in g[:3]])
    for a, b in zip(*res):
        assert torch.isfinite(b.float()).all()
        assert torch.equal(a, b)
