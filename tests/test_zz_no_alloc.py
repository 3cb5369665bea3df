"""hla_forward_noalloc (the forward pass on the library's fixed workspace
array) against hla_forward with a caller workspace, through the C ABI: two
calls in a row, the second smaller, each bit-identical to hla_forward (the
same kernels on the same inputs; the workspace's address is the only
difference) and within the stated tolerance of the fp64 oracle.  A call that
needs more than the array holds is refused before any work is enqueued."""
import numpy as np
import pytest

from causal_streaming_scans_amd import inputs as I
from hla_testlib import TOL, from_dev, oracle_forward, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


def _run_pair(variant, B, H, n, d, chunk, seg, seed, decay):
    import torch
    import causal_streaming_scans_amd as hla
    say(f"[noalloc] {variant} B={B} H={H} n={n} d={d} chunk={chunk} seg={seg}")
    dist = "uniform_pos" if variant.endswith("ratio") else "l2norm"
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist=dist, seed=seed, decay=decay)
    shp = (B, H, n, d)
    q, k, v = (to_dev(x[a], "bf16", shp) for a in "qkv")
    gamma = x["gamma"]
    need = hla.workspace_bytes(variant, B, H, n, d, d, chunk, seg)
    assert 0 < need <= hla.NOALLOC_SCRATCH_BYTES
    nst = B * H * hla.state_floats(variant, d, d)
    st_a = torch.empty(nst, dtype=torch.float32, device="cuda")
    st_b = torch.empty(nst, dtype=torch.float32, device="cuda")
    o_a = hla.hla_forward_noalloc(q, k, v, variant=variant, gamma=gamma, chunk=chunk,
                                  seg_chunks=seg, state_out=st_a)
    o_b = hla.hla_forward(q, k, v, variant=variant, gamma=gamma, chunk=chunk, seg_chunks=seg,
                          state_out=st_b)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    assert torch.equal(st_a, st_b)
    got = from_dev(o_a).reshape(B * H, n, d)
    want = oracle_forward(x, variant, H, gamma=gamma)
    err = rel_l2(got, want)
    say(f"   equal to hla_forward; oracle rel_l2 {err:.3e}")
    assert err < TOL["bf16"]


def test_noalloc_matches_forward_twice():
    # the benchmark's variant with many segments, then a smaller decayed call
    _run_pair("hla2_ratio", 2, 4, 1500, 64, 64, 2, 3100, False)
    _run_pair("hla2", 1, 2, 300, 64, 32, 2, 3101, True)


def test_noalloc_refuses_oversized_workspace():
    import torch
    import causal_streaming_scans_amd as hla
    B, H, n, d = 64, 16, 8192, 128
    need = hla.workspace_bytes("hla2", B, H, n, d, d, 16, 1)
    assert need > hla.NOALLOC_SCRATCH_BYTES
    q = torch.empty(1, dtype=torch.bfloat16, device="cuda")
    lib = hla.load()
    import ctypes
    P = ctypes.c_void_p
    rc = lib.hla_forward_noalloc(P(q.data_ptr()), P(q.data_ptr()), P(q.data_ptr()),
                                 P(q.data_ptr()), B, H, n, d, d, 1, 0, None, 16, 1, None, None,
                                 None)
    assert rc == 4   # HLA_ERR_WORKSPACE, before anything is enqueued
