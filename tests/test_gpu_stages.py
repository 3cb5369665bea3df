"""Stage-level parity: the workspace after stage 1 (segment summaries) and
after stage 2 (the up-sweep of the exclusive Blelloch scan) against the fp64
chunk-scan algebra of oracle/chunk_scan.py.

Layout (R = nseg - 1 summarised segments per head, parts X, Y, N, y, nv):
leaf s of head bh at slot bh*R + s; internal node (b >= 1, m), the combine of
segments m*2^b .. (m+1)*2^b - 1, at slot B*H*R + bh*R + (nodes of levels
1 .. b-1) + m, for every such node ending below R.  Stage 3's use of the
nodes is covered by the forward parity tests.
"""
import numpy as np
import pytest

from causal_streaming_scans_amd import inputs as I
from hla_testlib import TOL, rel_l2, say, to_dev
from oracle import chunk_scan as CS

pytestmark = pytest.mark.gpu


def _unpack(vec, d, dv):
    o = 0
    X = vec[o:o + d * d].reshape(d, d); o += d * d
    Y = vec[o:o + d * dv].reshape(d, dv); o += d * dv
    N = vec[o:o + d * dv].reshape(d, dv); o += d * dv
    y = vec[o:o + d]; o += d
    nv = vec[o:o + d]
    return X, Y, N, y, nv


def _ref_summaries(x, bh, variant, chunk, seg_len, nseg, g):
    q, k, v = (x[kk][bh].astype(np.float64) for kk in ("q", "k", "v"))
    sums = []
    for s in range(nseg):
        a, b = s * seg_len, min((s + 1) * seg_len, q.shape[0])
        if variant.startswith("hla2"):
            sm = CS.hla2_segment_summary(q[a:b], k[a:b], v[a:b], chunk, g)
            sums.append((sm["S"], sm["C"], sm["W"], sm["m"], sm["u"]))
        else:
            sm = CS.ahla_segment_summary(q[a:b], k[a:b], v[a:b], chunk, g)
            sums.append((sm["M"], sm["P"], sm["E"], sm["mK"], sm["nk"]))
    return sums


def _nodes(nreal):
    """(b, m, first segment, last segment, slot index within the head) of
    every internal node of the up-sweep."""
    out, off, b = [], 0, 1
    while (nreal >> b) > 0:
        for m in range(nreal >> b):
            out.append((b, m, m << b, ((m + 1) << b) - 1, off + m))
        off += nreal >> b
        b += 1
    return out


@pytest.mark.parametrize("dtype,variant,d,chunk,seg,decay", [
    ("f32", "hla2", 32, 16, 2, False),
    ("bf16", "hla2", 64, 64, 1, False),
    ("bf16", "hla2", 64, 64, 2, True),
    ("f32", "hla2", 64, 64, 2, True),
    ("bf16", "hla2", 64, 32, 2, False),
    ("bf16", "hla2", 64, 16, 4, True),
    ("bf16", "hla2", 128, 32, 2, True),
    ("bf16", "ahla", 64, 64, 1, False),
    ("bf16", "ahla", 64, 32, 2, False),
    ("f32", "ahla", 32, 16, 1, False),
    ("bf16", "ahla", 64, 64, 1, True),
    ("f32", "ahla", 32, 16, 2, True),
])
def test_summaries_and_up_sweep(dtype, variant, d, chunk, seg, decay):
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n = 1, 2, 9 * chunk * seg + 7          # 10 segments: nodes up to 8 wide
    say(f"[stages] {dtype} {variant} d={d} chunk={chunk} seg={seg} decay={decay} n={n}")
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="l2norm", seed=31, decay=decay)
    gam = x["gamma"]
    q = to_dev(x["q"], dtype, (B, H, n, d))
    k = to_dev(x["k"], dtype, (B, H, n, d))
    v = to_dev(x["v"], dtype, (B, H, n, d))
    nbytes = hla.workspace_bytes(variant, B, H, n, d, d, chunk, seg)
    ws = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    kw = dict(variant=variant, gamma=gam, chunk=chunk, seg_chunks=seg, workspace=ws)
    seg_len = chunk * seg
    nseg = -(-n // seg_len)
    nreal = nseg - 1
    sumf = d * d + 2 * d * d + 2 * d
    tol = TOL[dtype]
    worst = 0.0

    def slots():
        torch.cuda.synchronize()
        return ws.cpu().numpy().astype(np.float64).reshape(2 * B * H, nreal, sumf)

    hla.hla_forward_stage(1, q, k, v, **kw)
    e1 = slots()
    hla.hla_forward_stage(2, q, k, v, **kw)
    e = slots()
    for bh in range(B * H):
        g = 1.0 if gam is None else float(gam[bh % H])
        ref = _ref_summaries(x, bh, variant, chunk, seg_len, nseg, g)
        if variant.startswith("hla2"):
            items = [dict(S=r[0], C=r[1], W=r[2], m=r[3], u=r[4], l=seg_len) for r in ref]
            comb = lambda A, Bq: CS.hla2_combine(A, Bq, g)
            parts = lambda it: (it["S"], it["C"], it["W"], it["m"], it["u"])
        else:
            items = [dict(M=r[0], P=r[1], E=r[2], mK=r[3], nk=r[4], l=seg_len) for r in ref]
            comb = lambda A, Bq: CS.ahla_combine(A, Bq, g)
            parts = lambda it: (it["M"], it["P"], it["E"], it["mK"], it["nk"])
        for s_ in range(nreal):
            for stage_ws in (e1, e):      # the leaves are not touched by stage 2
                for name, a, b in zip(("X", "Y", "N", "y", "nv"), _unpack(stage_ws[bh, s_], d, d),
                                      parts(items[s_])):
                    err = rel_l2(a, b)
                    worst = max(worst, err)
                    assert err < tol, f"head {bh} summary {s_} part {name}: {err:.3e}"
        for (lev, m, lo, hi, idx) in _nodes(nreal):
            node = items[lo]
            for j in range(lo + 1, hi + 1):
                node = comb(node, items[j])
            got = _unpack(e[B * H + bh, idx], d, d)
            for name, a, b in zip(("X", "Y", "N", "y", "nv"), got, parts(node)):
                err = rel_l2(a, b)
                worst = max(worst, err)
                assert err < tol, f"head {bh} node ({lev},{m}) [{lo}..{hi}] part {name}: {err:.3e}"
    say(f"   {nreal} slots per head match, worst part rel_l2 {worst:.3e}")
