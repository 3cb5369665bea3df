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
