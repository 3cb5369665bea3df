"""Helpers shared by the GPU tests: run the HIP path and the oracle on the same
seeded inputs and compare them."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from causal_streaming_scans_amd import inputs as I

TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype, shape=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if shape is not None:
        t = t.reshape(shape)
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return t.cuda().contiguous()


def from_dev(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def worst_head(a, b):
    """Largest per-(b,h) relative L2 (diagnostic)."""
    a = np.asarray(a, np.float64).reshape(a.shape[0], -1)
    b = np.asarray(b, np.float64).reshape(b.shape[0], -1)
    num = np.linalg.norm(a - b, axis=1)
    den = np.maximum(np.linalg.norm(b, axis=1), 1e-300)
    return float((num / den).max())


def oracle_forward(x, variant, H, gamma=None, state_in=None, want_state=False, heads=None):
    """Oracle on all heads or on the listed head indices (bh)."""
    q, k, v = x["q"], x["k"], x["v"]
    if heads is not None:
        q, k, v = q[heads], k[heads], v[heads]
        if state_in is not None:
            state_in = state_in[heads]
    ratio = variant.endswith("ratio")
    if variant.startswith("hla2"):
        if heads is not None and gamma is not None:
            # per-head decays of the sampled heads, then H' = 1 per row
            gsel = np.asarray([gamma[h % H] for h in heads], np.float64)
            res = [oracle.hla2(q[i:i + 1], k[i:i + 1], v[i:i + 1], H=1, gamma=[gsel[i]],
                               ratio=ratio,
                               state_in=None if state_in is None else state_in[i:i + 1],
                               want_state=want_state) for i in range(len(heads))]
            if want_state:
                return (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]))
            return np.concatenate(res)
        return oracle.hla2(q, k, v, H=(1 if heads is not None else H), gamma=gamma, ratio=ratio,
                           state_in=state_in, want_state=want_state)
    if heads is not None and gamma is not None:
        gsel = [float(gamma[h % H]) for h in heads]
        res = [oracle.ahla(q[i:i + 1], k[i:i + 1], v[i:i + 1], ratio=ratio, H=1, gamma=[gsel[i]],
                           state_in=None if state_in is None else state_in[i:i + 1],
                           want_state=want_state) for i in range(len(heads))]
        if want_state:
            return (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]))
        return np.concatenate(res)
    return oracle.ahla(q, k, v, ratio=ratio, state_in=state_in, want_state=want_state,
                       H=(1 if heads is not None else H), gamma=gamma)


def gpu_forward(x, variant, B, H, dtype, chunk, seg_chunks=0, gamma=None, state_in=None,
                want_state=False):
    import torch
    import causal_streaming_scans_amd as hla
    n, d = x["q"].shape[1], x["q"].shape[2]
    dv = x["v"].shape[2]
    q = to_dev(x["q"], dtype, (B, H, n, d))
    k = to_dev(x["k"], dtype, (B, H, n, d))
    v = to_dev(x["v"], dtype, (B, H, n, dv))
    si = None
    if state_in is not None:
        si = torch.from_numpy(np.ascontiguousarray(state_in, np.float32)).cuda()
    so = None
    if want_state:
        so = torch.empty(B * H * hla.state_floats(variant, d, dv), dtype=torch.float32, device="cuda")
    o = hla.hla_forward(q, k, v, variant=variant, gamma=gamma, chunk=chunk, seg_chunks=seg_chunks,
                        state_in=si, state_out=so)
    torch.cuda.synchronize()
    out = from_dev(o).reshape(B * H, n, dv)
    if want_state:
        return out, so.cpu().numpy().astype(np.float64).reshape(B * H, -1)
    return out


def dgamma_scale(x, do, H, gamma, ratio):
    """Size of the terms of the decay gradient, per head h, from fp64 oracle
    tensors: (1/g_h) sum_{b,t} |t - c| (2|q.dq| + 3|z.dz| + |k.dk|/2), with
    Z = LA_g(Q, K, K), dz its full gradient, c = (n - 1)/2.  The terms sum to
    zero without the weight, so errors are judged against this size."""
    from oracle import backward as BW
    from oracle import definition as D
    BH, n, _ = x["q"].shape
    c = 0.5 * (n - 1)
    w = np.abs(np.arange(n) - c)
    out = np.zeros(H)
    for bh in range(BH):
        q, k, v = (np.asarray(x[a][bh], np.float64) for a in "qkv")
        dob = np.asarray(do[bh], np.float64)
        g = 1.0 if gamma is None else float(gamma[bh % H])
        dq, dk, _ = BW.hla2_vjp(q, k, v, dob, g, ratio)
        z = (D.decay_mask(n, g) * (q @ k.T)) @ k
        D2 = D.decay_mask(n, g * g)
        up = dob @ v.T
        if ratio:
            M = D2 * (q @ z.T)
            den = M.sum(axis=1, keepdims=True)
            o = (M @ v) / den
            up = (dob / den) @ v.T - (dob * o).sum(axis=1, keepdims=True) / den
        dz = (D2 * up).T @ q
        terms = 2 * np.abs((q * dq).sum(1)) + 3 * np.abs((z * dz).sum(1)) + 0.5 * np.abs((k * dk).sum(1))
        out[bh % H] += (w * terms).sum() / g
    return out
