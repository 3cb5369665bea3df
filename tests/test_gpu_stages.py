"""Stage-level parity: the workspace after each stage of the forward pass
against the fp64 chunk-scan algebra of oracle/chunk_scan.py.

Stage 1 writes the segment summaries (X, Y, N, y, nv per segment); stage 2
leaves the exclusive prefixes in the second half of the workspace.  Layout:
ws[bh][which][spad][summary floats], which = 0 (summaries), 1 (prefixes).
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
            sm = CS.ahla_segment_summary(q[a:b], k[a:b], v[a:b], chunk)
            sums.append((sm["M"], sm["P"], sm["E"], sm["mK"], sm["nk"]))
    return sums


@pytest.mark.parametrize("dtype,variant,d,chunk,seg,decay", [
    ("f32", "hla2", 32, 16, 2, False),
    ("bf16", "hla2", 64, 64, 1, False),
    ("bf16", "hla2", 64, 32, 2, False),
    ("bf16", "hla2", 64, 16, 4, True),
    ("bf16", "hla2", 128, 32, 2, True),
    ("bf16", "ahla", 64, 64, 1, False),
    ("bf16", "ahla", 64, 32, 2, False),
])
def test_summaries_and_prefixes(dtype, variant, d, chunk, seg, decay):
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n = 1, 2, 5 * chunk * seg + 7
    say(f"[stages] {dtype} {variant} d={d} chunk={chunk} seg={seg} decay={decay} n={n}")
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist="l2norm", seed=31, decay=decay)
    gam = x["gamma"]
    q = to_dev(x["q"], dtype, (B, H, n, d))
    k = to_dev(x["k"], dtype, (B, H, n, d))
    v = to_dev(x["v"], dtype, (B, H, n, d))
    nbytes = hla.workspace_bytes(variant, B, H, n, d, d, chunk, seg)
    ws = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    kw = dict(variant=variant, gamma=gam, chunk=chunk, seg_chunks=seg, workspace=ws)
    hla.hla_forward_stage(1, q, k, v, **kw)
    torch.cuda.synchronize()
    seg_len = chunk * seg
    nseg = -(-n // seg_len)
    spad = 1
    while spad < nseg:
        spad *= 2
    sumf = d * d + 2 * d * d + 2 * d
    e = ws.cpu().numpy().astype(np.float64).reshape(B * H, 2, spad, sumf)
    tol = 10 * TOL[dtype]
    for bh in range(B * H):
        g = 1.0 if gam is None else float(gam[bh % H])
        ref = _ref_summaries(x, bh, variant, chunk, seg_len, nseg, g)
        for s in range(nseg - 1):
            got = _unpack(e[bh, 0, s], d, d)
            for name, a, b in zip(("X", "Y", "N", "y", "nv"), got, ref[s]):
                err = rel_l2(a, b)
                assert err < tol, f"summary head {bh} seg {s} part {name}: {err:.3e}"
    hla.hla_forward_stage(2, q, k, v, **kw)
    torch.cuda.synchronize()
    e = ws.cpu().numpy().astype(np.float64).reshape(B * H, 2, spad, sumf)
    for bh in range(B * H):
        g = 1.0 if gam is None else float(gam[bh % H])
        ref = _ref_summaries(x, bh, variant, chunk, seg_len, nseg, g)
        if variant.startswith("hla2"):
            items = [dict(S=r[0], C=r[1], W=r[2], m=r[3], u=r[4], l=seg_len) for r in ref]
            pref = CS.blelloch_exclusive(items, lambda A, Bq: CS.hla2_combine(A, Bq, g),
                                         lambda: CS.hla2_zero(d, d))
            want = [(p["S"], p["W"], p["u"]) for p in pref]
            parts = (0, 2, 4)
        else:
            items = [dict(M=r[0], P=r[1], E=r[2], mK=r[3], nk=r[4]) for r in ref]
            pref = CS.blelloch_exclusive(items, CS.ahla_combine, lambda: CS.ahla_zero(d, d))
            want = [(p["P"], p["E"], p["mK"], p["nk"]) for p in pref]
            parts = (1, 2, 3, 4)
        for s in range(1, nseg):
            got = _unpack(e[bh, 1, s], d, d)
            for j, pidx in enumerate(parts):
                err = rel_l2(got[pidx], want[s][j])
                assert err < tol, f"prefix head {bh} seg {s} part {pidx}: {err:.3e}"
    say("   summaries and prefixes match")
