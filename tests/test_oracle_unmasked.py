"""Pins for the unmasked operators of oracle/unmasked.py: the matrix form
against explicit triple sums, a closed form, homogeneity, permutation
equivariance (no mask: reordering the tokens reorders the outputs, which the
causal operators do not do), and the moment factorisation the pages state
for the unmasked product ("Resumen Tecnico: Atencion Lineal de Orden
Superior (HLA)", gist.science/es/paper/2510.27258, sections "1. HLA de
Segundo Orden" and "2. ... (AHLA)")."""
import numpy as np
import pytest

from oracle import unmasked as U
from oracle import definition as D


def _inputs(seed, n=7, d=3, dv=2):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, dv))


@pytest.mark.parametrize("variant", ["hla2", "ahla"])
def test_matrix_equals_loops(variant):
    q, k, v = _inputs(1)
    mat = U.hla2_unmasked if variant == "hla2" else U.ahla_unmasked
    loops = U.hla2_unmasked_loops if variant == "hla2" else U.ahla_unmasked_loops
    assert np.allclose(mat(q, k, v), loops(q, k, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("variant", ["hla2", "ahla"])
def test_all_ones_closed_form(variant):
    """d = 1, q = k = v = 1: every A entry is 1, so o_t = n^2 for both."""
    n = 9
    one = np.ones((n, 1))
    mat = U.hla2_unmasked if variant == "hla2" else U.ahla_unmasked
    assert np.allclose(mat(one, one, one), n * n)


@pytest.mark.parametrize("variant", ["hla2", "ahla"])
def test_homogeneity_and_permutation(variant):
    q, k, v = _inputs(2, n=11)
    mat = U.hla2_unmasked if variant == "hla2" else U.ahla_unmasked
    o = mat(q, k, v)
    assert np.allclose(mat(2 * q, k, v), 4 * o)     # degree 2 in q
    assert np.allclose(mat(q, 2 * k, v), 4 * o)     # degree 2 in k
    assert np.allclose(mat(q, k, 3 * v), 3 * o)     # linear in v
    perm = np.random.default_rng(3).permutation(11)
    assert np.allclose(mat(q[perm], k[perm], v[perm]), o[perm])
    # the masked operators are not equivariant
    masked = D.hla2_matrix(q, k, v) if variant == "hla2" else D.ahla_matrix(q, k, v)
    masked_p = D.hla2_matrix(q[perm], k[perm], v[perm]) if variant == "hla2" \
        else D.ahla_matrix(q[perm], k[perm], v[perm])
    assert not np.allclose(masked_p, masked[perm])


def test_moment_factorisation():
    """The unmasked product is the product of whole-sequence moments:
    HLA-2 q^T (K^T K)(Q^T V), AHLA q^T (K^T Q)(K^T V)."""
    q, k, v = _inputs(4, n=13, d=4, dv=3)
    assert np.allclose(U.hla2_unmasked(q, k, v), q @ (k.T @ k) @ (q.T @ v))
    assert np.allclose(U.ahla_unmasked(q, k, v), q @ (k.T @ q) @ (k.T @ v))


def test_planted_mistakes_are_caught():
    """A transposed factor or the wrong operand order moves the result far
    from the loops: HLA-2 with A A in place of A A^T, AHLA with A^T A."""
    q, k, v = _inputs(5, n=8, d=3, dv=2)
    A = q @ k.T
    ref2, refa = U.hla2_unmasked_loops(q, k, v), U.ahla_unmasked_loops(q, k, v)
    for wrong, ref in ((A @ (A @ v), ref2), (A.T @ (A @ v), refa), (A @ (A.T @ v), refa)):
        assert np.linalg.norm(wrong - ref) > 1e-3 * np.linalg.norm(ref)
