"""Pins for the third-order oracle (oracle/third_order.py), page section "3.
HLA de Tercer Orden" of "Resumen Tecnico: Atencion Lineal de Orden Superior
(HLA)" (gist.science/es/paper/2510.27258): its three forms against each
other, a closed form, the unmasked moment product the page names, the
chained reduction through the second-order definition, homogeneity and
causality."""
import numpy as np
import pytest

from oracle import definition as D
from oracle import third_order as T3


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rnd(seed, n, d, dv):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, d)) / np.sqrt(d), rng.standard_normal((n, d)) / np.sqrt(d),
            rng.standard_normal((n, dv)))


def test_loops_matrix_serial_agree():
    q, k, v = rnd(1, 9, 3, 2)
    a = T3.hla3_loops(q, k, v)
    assert rel(T3.hla3_matrix(q, k, v), a) < 1e-13
    assert rel(T3.hla3_serial(q, k, v), a) < 1e-13
    q, k, v = rnd(2, 150, 8, 5)
    assert rel(T3.hla3_serial(q, k, v), T3.hla3_matrix(q, k, v)) < 1e-12


def test_all_ones_closed_form():
    """q = k = v = 1 (d = dv = 1): o_t = sum_{m<=t} (m+1)^2 = (t+1)(t+2)(2t+3)/6."""
    n = 40
    one = np.ones((n, 1))
    t = np.arange(n)
    want = (t + 1) * (t + 2) * (2 * t + 3) / 6
    np.testing.assert_allclose(T3.hla3_loops(one[:8], one[:8], one[:8])[:, 0], want[:8], rtol=0)
    np.testing.assert_allclose(T3.hla3_matrix(one, one, one)[:, 0], want, rtol=1e-15)
    np.testing.assert_allclose(T3.hla3_serial(one, one, one)[:, 0], want, rtol=1e-15)


def test_unmasked_moments():
    """Without masks the product is q_t^T S^K S^Q P^KV over the whole
    sequence; the masked output at the last token differs from it only by the
    pairs the masks remove, so check the unmasked algebra directly."""
    q, k, v = rnd(3, 30, 4, 3)
    A = q @ k.T
    full = A @ A.T @ A @ v
    SK, SQ, PKV = k.T @ k, q.T @ q, k.T @ v
    assert rel(q @ SK @ SQ @ PKV, full) < 1e-13
    # and the masked operator is not the unmasked one (the masks matter)
    assert rel(T3.hla3_matrix(q, k, v), full) > 1e-2


def test_chained_reduction():
    """o = HLA-2(Q, K, Y) with Y = tril(Q K^T) V, through the second-order
    brute-force definition (oracle/definition.py) and a first-order causal
    linear attention written here."""
    q, k, v = rnd(4, 70, 6, 4)
    y = np.tril(q @ k.T) @ v
    assert rel(D.hla2_matrix(q, k, y), T3.hla3_matrix(q, k, v)) < 1e-12


def test_homogeneity_and_causality():
    q, k, v = rnd(5, 60, 5, 3)
    o = T3.hla3_matrix(q, k, v)
    assert rel(T3.hla3_matrix(2 * q, 3 * k, 0.5 * v), (8 * 27 * 0.5) * o) < 1e-13
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[40:] += 1
    k2[40:] -= 2
    v2[40:] *= 3
    assert rel(T3.hla3_matrix(q2, k2, v2)[:40], o[:40]) < 1e-14


def test_other_mask_placements_are_not_causal():
    """The placements the docstring rejects read future tokens: changing a
    later token changes an earlier output."""
    q, k, v = rnd(6, 20, 3, 2)

    def no_inner(q, k, v):
        L = np.tril(q @ k.T)
        return np.tril(L @ L.T @ L) @ v

    q2 = q.copy()
    q2[15] += 1.0
    assert not np.allclose(no_inner(q2, k, v)[:10], no_inner(q, k, v)[:10])
    assert np.allclose(T3.hla3_matrix(q2, k, v)[:15], T3.hla3_matrix(q, k, v)[:15], rtol=1e-14)
