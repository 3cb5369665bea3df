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


# ------------------------------------------------- decay and the ratio form

def _la(q, k, v, g=1.0):
    """Textbook causal linear attention with decay, by its own recurrence:
    M <- g M + k v^T, out_t = M^T q_t."""
    M = np.zeros((q.shape[1], v.shape[1]))
    out = np.empty((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        M = g * M + np.outer(k[t], v[t])
        out[t] = q[t] @ M
    return out


@pytest.mark.parametrize("gamma", [1.0, 0.8, 0.95])
@pytest.mark.parametrize("ratio", [False, True])
def test_decay_and_ratio_forms_agree(gamma, ratio):
    rng = np.random.default_rng(41)
    q, k, v = rng.random((9, 3)), rng.random((9, 3)), rng.standard_normal((9, 2))
    a = T3.hla3_loops(q, k, v, gamma, ratio)
    assert rel(T3.hla3_matrix(q, k, v, gamma, ratio), a) < 1e-13
    assert rel(T3.hla3_serial(q, k, v, gamma, ratio), a) < 1e-13
    q, k, v = rng.random((120, 6)) / 6, rng.random((120, 6)) / 6, rng.standard_normal((120, 4))
    assert rel(T3.hla3_serial(q, k, v, gamma, ratio), T3.hla3_matrix(q, k, v, gamma, ratio)) < 1e-12


@pytest.mark.parametrize("gamma", [0.5, 0.9])
def test_decay_all_ones_closed_form(gamma):
    """q = k = v = 1 (d = dv = 1): the weight of (i, m, j) is
    g^((t-i)+(t-m)+(t-j)), so o_t = sum_{m<=t} g^(3(t-m)) (sum_{i<=m} g^(m-i))^2
    = sum_{m<=t} g^(3(t-m)) ((1 - g^(m+1)) / (1 - g))^2."""
    n = 30
    one = np.ones((n, 1))
    want = [sum(gamma ** (3 * (t - m)) * ((1 - gamma ** (m + 1)) / (1 - gamma)) ** 2
                for m in range(t + 1)) for t in range(n)]
    np.testing.assert_allclose(T3.hla3_serial(one, one, one, gamma)[:, 0], want, rtol=1e-13)
    np.testing.assert_allclose(T3.hla3_loops(one[:7], one[:7], one[:7], gamma)[:, 0], want[:7],
                               rtol=1e-13)


@pytest.mark.parametrize("gamma", [1.0, 0.9])
def test_decay_is_chained_linear_attention(gamma):
    """o = LA_{g^3}(Q, LA_g(Q, K, K), LA_g(Q, K, V)): keys z_m = S_m q_m and
    values y_m = P_m^T q_m, each decayed to m, meet with g^(3(t-m))."""
    q, k, v = rnd(42, 60, 5, 3)
    want = _la(q, _la(q, k, k, gamma), _la(q, k, v, gamma), gamma ** 3)
    assert rel(T3.hla3_serial(q, k, v, gamma), want) < 1e-12


def test_decay_zero_and_ratio_invariants():
    q, k, v = rnd(43, 25, 4, 3)
    # g = 0 keeps i = m = j = t only: o_t = (q_t . k_t)^3 v_t
    want = ((q * k).sum(1) ** 3)[:, None] * v
    assert rel(T3.hla3_serial(q, k, v, 0.0), want) < 1e-13
    rng = np.random.default_rng(44)
    qp, kp = rng.random((30, 4)), rng.random((30, 4))
    c = np.ones((30, 3)) * np.array([0.5, -1.0, 3.0])
    assert rel(T3.hla3_serial(qp, kp, c, 0.9, ratio=True), c) < 1e-13
    # the ratio form is homogeneous of degree 0 in q and in k
    vp = rng.standard_normal((30, 3))
    base = T3.hla3_serial(qp, kp, vp, 0.9, ratio=True)
    assert rel(T3.hla3_serial(2.5 * qp, 0.3 * kp, vp, 0.9, ratio=True), base) < 1e-13


def test_decay_causality_and_resume():
    q, k, v = rnd(45, 50, 4, 3)
    o1 = T3.hla3_serial(q, k, v, 0.9, ratio=False)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[30:] += 1.0
    v2[30:] *= -2.0
    o2 = T3.hla3_serial(q2, k2, v2, 0.9)
    assert np.array_equal(o1[:30], o2[:30])
    for ratio in (False, True):
        qq, kk = (np.abs(q), np.abs(k)) if ratio else (q, k)
        whole = T3.hla3_serial(qq, kk, v, 0.93, ratio)
        a, st = T3.hla3_serial_state(qq[:21], kk[:21], v[:21], 0.93, ratio)
        b, _ = T3.hla3_serial_state(qq[21:], kk[21:], v[21:], 0.93, ratio, state=st)
        assert rel(np.concatenate([a, b]), whole) < 1e-13


def test_decay_law_rejects_plausible_mistakes():
    """The second-order weight law g^((t-i)+(t-j)) (no term for m), and g^2
    instead of g^3 between the keys' and values' chains, each differ from the
    reading far beyond the tolerances above."""
    q, k, v = rnd(46, 20, 4, 3)
    g = 0.85
    good = T3.hla3_serial(q, k, v, g)
    assert rel(_la(q, _la(q, k, k, g), _la(q, k, v, g), g ** 2), good) > 1e-2
    n = q.shape[0]
    A = q @ k.T
    bad = np.zeros_like(good)
    for t in range(n):
        for m in range(t + 1):
            for i in range(m + 1):
                for j in range(m + 1):
                    bad[t] += g ** ((t - i) + (t - j)) * A[t, i] * A[m, i] * A[m, j] * v[j]
    assert rel(bad, good) > 1e-2


@pytest.mark.parametrize("gamma,ratio", [(1.0, False), (0.8, False), (0.9, True)])
def test_backward_by_central_differences_and_euler(gamma, ratio):
    rng = np.random.default_rng(47)
    n, d, dv = 8, 3, 2
    q, k = (rng.random((n, d)), rng.random((n, d))) if ratio else \
        (rng.standard_normal((n, d)), rng.standard_normal((n, d)))
    v = rng.standard_normal((n, dv))
    do = rng.standard_normal((n, dv))
    dq, dk, dv_ = T3.hla3_vjp(q, k, v, do, gamma, ratio)
    h = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv_)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            fp = (T3.hla3_matrix(q, k, v, gamma, ratio) * do).sum()
            x[idx] = x0 - h
            fm = (T3.hla3_matrix(q, k, v, gamma, ratio) * do).sum()
            x[idx] = x0
            num[idx] = (fp - fm) / (2 * h)
        assert rel(dx, num) < 1e-6
    # Euler: o has degree 3 in q, 3 in k, 1 in v (ratio: 0, 0, 1)
    o = T3.hla3_matrix(q, k, v, gamma, ratio)
    ref = float((do * o).sum())
    dq_deg = 0 if ratio else 3
    np.testing.assert_allclose(float((q * dq).sum()), dq_deg * ref, atol=1e-9 * abs(ref) + 1e-12)
    np.testing.assert_allclose(float((v * dv_).sum()), ref, rtol=1e-10)
