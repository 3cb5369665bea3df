"""GPU parity of hla_unmasked_forward (the unmasked operators (A A^T) V and
(A A) V, A = Q K^T) against the fp64 oracle of oracle/unmasked.py, on the
operators of "1. HLA de Segundo Orden" and "2. ... (AHLA)" without their masks
("Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
gist.science/es/paper/2510.27258).  Relative L2 per head: 1e-5 fp32, 1e-2
bf16 (the oracle consumes the same bf16-rounded inputs)."""
import numpy as np
import pytest

from oracle import unmasked as U
from causal_streaming_scans_amd import inputs as I
from hla_testlib import TOL, from_dev, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


def run(x, variant, B, H, dtype):
    import torch
    import causal_streaming_scans_amd as hla
    n, d = x["q"].shape[1], x["q"].shape[2]
    shp = (B, H, n, d)
    o = hla.hla_unmasked_forward(*(to_dev(x[a], dtype, shp) for a in "qkv"), variant=variant)
    torch.cuda.synchronize()
    return from_dev(o).reshape(B * H, n, d)


CASES = [
    # dtype, variant, B, H, n, d, dist
    ("f32", "hla2", 1, 2, 300, 16, "normal_scaled"),
    ("f32", "hla2", 2, 1, 33, 32, "normal_scaled"),
    ("f32", "ahla", 1, 2, 257, 64, "normal_scaled"),
    ("f32", "hla2", 1, 1, 1, 64, "normal_scaled"),
    ("f32", "ahla", 1, 2, 200, 128, "normal_scaled"),
    ("bf16", "hla2", 2, 2, 777, 64, "l2norm"),
    ("bf16", "ahla", 1, 3, 500, 64, "l2norm"),
    ("bf16", "hla2", 1, 2, 450, 128, "l2norm"),
    ("bf16", "ahla", 1, 2, 65, 16, "l2norm"),
    ("bf16", "hla2", 1, 2, 31, 32, "l2norm"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_unmasked_matches_oracle(case):
    dtype, variant, B, H, n, d, dist = case
    say(f"[unmasked] {case}")
    x = I.make_inputs(B, H, n, d, d, dtype=dtype, dist=dist, seed=1300 + n + d)
    got = run(x, variant, B, H, dtype)
    want = U.unmasked_batched(x["q"], x["k"], x["v"], variant)
    for bh in range(B * H):
        e = rel_l2(got[bh], want[bh])
        say(f"  head {bh}: rel_l2 {e:.3e}")
        assert e < TOL[dtype], (case, bh, e)


@pytest.mark.parametrize("variant", ["hla2", "ahla"])
def test_unmasked_benchmark_shape_sampled_heads(variant):
    """B=8 H=16 n=4096 d=64 bf16 (the benchmark's shape), q, k L2-normalised
    Gaussian rows, v ~ N(0,1); the oracle on the first and last head."""
    B, H, n, d = 8, 16, 4096, 64
    say(f"[unmasked] {variant} B={B} H={H} n={n} d={d} bf16")
    x = I.make_inputs(B, H, n, d, d, dtype="bf16", dist="l2norm", seed=1400)
    got = run(x, variant, B, H, "bf16")
    heads = [0, B * H - 1]
    want = U.unmasked_batched(x["q"], x["k"], x["v"], variant, heads=heads)
    for i, bh in enumerate(heads):
        e = rel_l2(got[bh], want[i])
        say(f"  head {bh}: rel_l2 {e:.3e}")
        assert e < TOL["bf16"]
