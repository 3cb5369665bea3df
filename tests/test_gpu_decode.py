"""Decode step (hla_step) vs the oracle: a forward pass over the first n
tokens hands its state_out to T single-token steps; every step's output and
the final state must match the oracle run over all n + T tokens.  Covers
every variant (HLA-2 with a per-head decay) at fp32 and bf16 head sizes."""
import numpy as np
import pytest

from causal_streaming_scans_amd import inputs as I
from hla_testlib import TOL, from_dev, gpu_forward, oracle_forward, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant,decay", [("hla2", True), ("hla2_ratio", True), ("ahla", False),
                                           ("ahla_ratio", False), ("ahla", True),
                                           ("ahla_ratio", True)])
@pytest.mark.parametrize("dtype,d", [("f32", 16), ("f32", 32), ("bf16", 64), ("bf16", 128)])
def test_decode_continues_forward(variant, decay, dtype, d):
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n, T = 2, 2, 100, 20
    ratio = variant.endswith("ratio")
    say(f"[decode] {variant} decay={decay} {dtype} d={d} n={n} T={T}")
    x = I.make_inputs(B, H, n + T, d, d, dtype=dtype,
                      dist="uniform_pos" if ratio else "normal_scaled", seed=900 + d, decay=decay)
    g = x["gamma"]
    head = {kk: x[kk][:, :n] for kk in ("q", "k", "v")}
    _, st = gpu_forward(head, variant, B, H, dtype, 32, 2, gamma=g, want_state=True)
    state = torch.from_numpy(np.ascontiguousarray(st, np.float32)).cuda().reshape(-1)
    outs = []
    for t in range(T):
        qd = to_dev(x["q"][:, n + t], dtype, (B, H, d))
        kd = to_dev(x["k"][:, n + t], dtype, (B, H, d))
        vd = to_dev(x["v"][:, n + t], dtype, (B, H, d))
        outs.append(from_dev(hla.hla_step(qd, kd, vd, state, variant=variant, gamma=g)))
    torch.cuda.synchronize()
    got = np.stack(outs, axis=2).reshape(B * H, T, d)   # [B, H, T, d]
    want, wst = oracle_forward(x, variant, H, gamma=g, want_state=True)
    err = rel_l2(got, want[:, n:])
    serr = rel_l2(state.cpu().numpy().astype(np.float64).reshape(B * H, -1), wst)
    say(f"   decode rel_l2 {err:.3e}  state rel_l2 {serr:.3e}")
    assert np.isfinite(got).all()
    assert err < TOL[dtype]
    assert serr < TOL[dtype]
