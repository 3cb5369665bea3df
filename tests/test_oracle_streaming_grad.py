"""Pins for the oracle's linear-time gradients (oracle/streaming_grad.py).

They restate the HLA-2 and AHLA gradients as chains of causal linear
attention ("1. HLA de Segundo Orden" and "2. ... (AHLA)" of "Resumen
Tecnico: Atencion Lineal de Orden Superior (HLA)",
gist.science/es/paper/2510.27258).  Pinned here to things other than
themselves: the two sums they are built from against explicit double sums,
and every gradient element against the matrix-form chain rule of
oracle/backward.py (itself pinned by central differences), with and without
decay and the ratio form; a planted mistake in the gradient rule fails."""
import numpy as np
import pytest

from oracle import backward as BW
from oracle import streaming_grad as SG

from test_oracle_pins import rand_qkv, rel


def _brute_la(a, b, c, g):
    n = a.shape[0]
    out = np.zeros((n, c.shape[1]))
    for t in range(n):
        for s in range(t + 1):
            out[t] += g ** (t - s) * float(a[t] @ b[s]) * c[s]
    return out


def _brute_rla(x, y, z, g):
    n = x.shape[0]
    out = np.zeros((n, z.shape[1]))
    for s in range(n):
        for t in range(s, n):
            out[s] += g ** (t - s) * float(x[s] @ y[t]) * z[t]
    return out


@pytest.mark.parametrize("g", [1.0, 0.8])
def test_sums_equal_double_sums(g):
    rng = np.random.default_rng(41)
    a, b = rng.standard_normal((2, 3, 13, 4))
    c = rng.standard_normal((3, 13, 2))
    gg = np.full(3, g)
    got = SG.causal_la(a, b, c, gg)
    got_r = SG.anti_causal_la(a, b, c, gg)
    for h in range(3):
        assert rel(got[h], _brute_la(a[h], b[h], c[h], g)) < 1e-14
        assert rel(got_r[h], _brute_rla(a[h], b[h], c[h], g)) < 1e-14


@pytest.mark.parametrize("n", [1, 2, 29])
@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("ratio", [False, True])
@pytest.mark.parametrize("variant", ["hla2", "ahla"])
def test_equals_matrix_chain_rule(variant, ratio, decay, n):
    rng = np.random.default_rng(42 + n)
    H, B = 2, 2
    q, k, v = rand_qkv(rng, B * H, n, 5, 3, pos=ratio)
    do = rng.standard_normal(v.shape)
    gamma = np.array([0.9, 0.97]) if decay else None
    if variant == "hla2":
        got = SG.hla2_vjp_streaming(q, k, v, do, H, gamma, ratio)
        want = BW.hla2_vjp_batched(q, k, v, do, H, gamma, ratio)
    else:
        got = SG.ahla_vjp_streaming(q, k, v, do, H, gamma, ratio)
        want = BW.ahla_vjp_batched(q, k, v, do, ratio, H=H, gamma=gamma)
    for a, b in zip(got, want):
        assert a.shape == b.shape
        # with one token the ratio form's q, k gradients vanish (o = v):
        # both sides are then rounding noise, compared on an absolute scale
        assert np.linalg.norm(a - b) <= 1e-12 * max(np.linalg.norm(b), 1e-2)


def test_planted_mistake_fails():
    """Keys and values swapped in the key gradient's sum (RLA(a, dout, c)
    instead of RLA(c, dout, a)) differs from the chain rule far beyond the
    1e-12 above."""
    rng = np.random.default_rng(43)
    q, k, v = rand_qkv(rng, 1, 20, 4, 4)
    do = rng.standard_normal(v.shape)
    orig = SG.la_vjp

    def wrong(a, b, c, dout, g):
        return (SG.causal_la(dout, c, b, g), SG.anti_causal_la(a, dout, c, g),
                SG.anti_causal_la(b, a, dout, g))
    SG.la_vjp = wrong
    try:
        got = SG.hla2_vjp_streaming(q, k, v, do)
    finally:
        SG.la_vjp = orig
    want = BW.hla2_vjp_batched(q, k, v, do, 1)
    assert rel(got[1], want[1]) > 1e-2
