"""HLA through PyTorch autograd (causal_streaming_scans_amd.layer): the
differentiable operator and the attention sub-layer, against references built
only from the fp64 oracle (the masked definitions of oracle/definition.py and
the chain-rule gradients of oracle/backward.py) and the chain rule through the
projections written out in NumPy.  The drop-in sub-layer is the pages' use of
HLA ("Significancia" of "Resumen Tecnico: Atencion Lineal de Orden Superior
(HLA)", gist.science/es/paper/2510.27258)."""
import numpy as np
import pytest

from causal_streaming_scans_amd import inputs as I
from oracle import backward as BW
from oracle import definition as D
from hla_testlib import TOL, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["hla2", "hla2_ratio", "ahla"])
def test_hla_function_gradients(variant):
    import torch
    from causal_streaming_scans_amd.layer import hla
    B, H, n, d = 1, 2, 300, 64
    say(f"[autograd] {variant} B={B} H={H} n={n} d={d} bf16")
    dist = "uniform_pos" if variant.endswith("ratio") else "l2norm"
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist=dist, seed=1201, decay=variant == "hla2")
    gamma = x["gamma"] if variant == "hla2" else None
    q, k, v = (to_dev(x[key], "bf16", (B, H, n, d)).requires_grad_() for key in ("q", "k", "v"))
    w = I.make_upstream_grad(B * H, n, d, "bf16", seed=1202)
    o = hla(q, k, v, variant, gamma)
    (o.float() * torch.from_numpy(w).reshape(B, H, n, d).cuda()).sum().backward()
    torch.cuda.synchronize()
    if variant.startswith("hla2"):
        want = BW.hla2_vjp_batched(x["q"], x["k"], x["v"], w, H, gamma, ratio=variant.endswith("ratio"))
    else:
        want = BW.ahla_vjp_batched(x["q"], x["k"], x["v"], w)
    for name, t, ref in zip(("q", "k", "v"), (q, k, v), want):
        e = rel_l2(t.grad.float().cpu().numpy().reshape(ref.shape), ref)
        say(f"  d{name}: rel_l2 {e:.3e}")
        assert e < TOL["bf16"]


def _reference(xin, W, variant, H, hd, gy, gamma=None):
    """fp64 forward and gradients of the sub-layer from the oracle."""
    Wq, Wk, Wv, Wo = W
    B, n, _ = xin.shape

    def split(t):                               # [B, n, H*hd] -> [B*H, n, hd]
        return t.reshape(B, n, H, hd).transpose(0, 2, 1, 3).reshape(B * H, n, hd)

    def merge(t):
        return t.reshape(B, H, n, hd).transpose(0, 2, 1, 3).reshape(B, n, H * hd)

    q, k, v = split(xin @ Wq.T), split(xin @ Wk.T), split(xin @ Wv.T)
    if variant == "hla2":
        o = D.hla2_batched(q, k, v, H, gamma)
    else:
        o = D.ahla_batched(q, k, v)
    om = merge(o)
    y = om @ Wo.T
    dom = gy @ Wo
    dWo = np.einsum("bni,bnj->ij", gy, om)
    do = split(dom)
    if variant == "hla2":
        dq, dk, dv = BW.hla2_vjp_batched(q, k, v, do, H, gamma)
    else:
        dq, dk, dv = BW.ahla_vjp_batched(q, k, v, do)
    dq, dk, dv = merge(dq), merge(dk), merge(dv)
    dx = dq @ Wq + dk @ Wk + dv @ Wv
    grads = [np.einsum("bni,bnj->ij", g, xin) for g in (dq, dk, dv)] + [dWo]
    return y, dx, grads


@pytest.mark.parametrize("dtype,variant", [("f32", "hla2"), ("f32", "ahla"), ("bf16", "hla2"),
                                           ("bf16", "ahla")])
def test_sublayer(dtype, variant):
    """Output, input gradient and the four weight gradients of HLAAttention."""
    import torch
    from causal_streaming_scans_amd.layer import HLAAttention
    B, n, dm, H, hd = 2, 200, 96, 3, 32
    say(f"[sub-layer] {variant} {dtype} B={B} n={n} d_model={dm} heads={H} head_dim={hd}")
    rng = np.random.default_rng(1301)
    rnd = I.bf16_round if dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    xin = rnd((rng.standard_normal((B, n, dm)) / np.sqrt(dm)).astype(np.float32))
    W = [rnd((rng.standard_normal(s) / np.sqrt(s[1])).astype(np.float32))
         for s in ((H * hd, dm), (H * hd, dm), (H * hd, dm), (dm, H * hd))]
    gy = rnd(rng.standard_normal((B, n, dm)).astype(np.float32))
    gamma = np.asarray([0.97, 0.99, 0.995], np.float32) if variant == "hla2" else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    layer = HLAAttention(dm, H, hd, variant=variant, gamma=gamma, device="cuda", dtype=tdt)
    with torch.no_grad():
        for lin, w in zip((layer.wq, layer.wk, layer.wv, layer.wo), W):
            lin.weight.copy_(torch.from_numpy(w))
    x = torch.from_numpy(xin).to("cuda", tdt).requires_grad_()
    y = layer(x)
    y.backward(torch.from_numpy(gy).to("cuda", tdt))
    torch.cuda.synchronize()
    y_ref, dx_ref, g_ref = _reference(xin.astype(np.float64), [w.astype(np.float64) for w in W],
                                      variant, H, hd, gy.astype(np.float64), gamma)
    # the projections round q, k, v, o to the layer's dtype before the next
    # product: the bf16 layer measured 3.6-5.3e-3, inside the operator's bar
    tol = TOL[dtype]
    got = [("y", y, y_ref), ("dx", x.grad, dx_ref)] + \
          [(f"d{nm}", lin.weight.grad, r) for nm, lin, r in
           zip(("Wq", "Wk", "Wv", "Wo"), (layer.wq, layer.wk, layer.wv, layer.wo), g_ref)]
    for name, t, ref in got:
        e = rel_l2(t.detach().float().cpu().numpy(), ref)
        say(f"  {name}: rel_l2 {e:.3e}")
        assert e < tol, (name, e)


def test_learned_decay_gradient():
    """A decay tensor that requires grad receives dL/dgamma through autograd:
    the library's decay gradient against the oracle's chain rule, relative
    to itself and to the size of its terms (fp32)."""
    import torch
    from causal_streaming_scans_amd.layer import hla
    from hla_testlib import dgamma_scale
    B, H, n, d = 2, 3, 257, 32
    say(f"[autograd] learned decay B={B} H={H} n={n} d={d} fp32")
    x = I.make_inputs(B, H, n, d, d, dtype="f32", dist="l2norm", seed=1211, decay=True)
    q, k, v = (to_dev(x[key], "f32", (B, H, n, d)) for key in ("q", "k", "v"))
    gamma = torch.tensor(x["gamma"], dtype=torch.float32, requires_grad=True)
    w = I.make_upstream_grad(B * H, n, d, "f32", seed=1212)
    o = hla(q, k, v, "hla2", gamma)
    (o * torch.from_numpy(w).reshape(B, H, n, d).cuda()).sum().backward()
    torch.cuda.synchronize()
    want = BW.hla2_dgamma_batched(x["q"], x["k"], x["v"], w, H, x["gamma"])
    got = gamma.grad.double().numpy()
    scale = dgamma_scale(x, w, H, x["gamma"], False)
    rel = np.abs(got - want) / np.abs(want)
    say(f"  dgamma {got} want {want} rel {rel} err/scale {np.abs(got - want) / scale}")
    assert np.all(rel < TOL["f32"])
    assert np.all(np.abs(got - want) <= TOL["f32"] * scale)
