"""Pins for the oracle's AHLA with exponential decay.

Reading ("Contribuciones Clave", item 2 of "Resumen Tecnico: Atencion Lineal
de Orden Superior (HLA)", gist.science/es/paper/2510.27258, names masked
operators with and without decay; section "2. ... (AHLA)" names the
summaries P^KV, E, m^K, n): every streaming summary decays by g per token,
as for HLA-2, so the term A[t,i] A[i,j] v_j of o_t carries g^(t-j):
o = ((D_g * L)(D_g * L)) V = LA_g(Q, K, LA_g(Q, K, V)).  The pages fix no
decay law, so this is pinned to its own definition written three
independent ways (loops, matrix, textbook decayed linear attention twice),
to a hand-derived closed form, to its g = 0 and g = 1 special cases, to the
exact scan, and against plausible mistakes -- not to the pages."""
import numpy as np
import pytest

import oracle
from oracle import backward as BW
from oracle import chunk_scan as CS
from oracle import definition as D

from test_oracle_pins import _causal_la, rand_qkv, rel


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_lib):
    return oracle_lib


@pytest.mark.parametrize("gamma", [0.0, 0.5, 0.93, 1.0])
@pytest.mark.parametrize("ratio", [False, True])
def test_matrix_equals_loops(gamma, ratio):
    rng = np.random.default_rng(31)
    q, k, v = (x[0] for x in rand_qkv(rng, 1, 11, 3, 2, pos=True))
    assert rel(D.ahla_matrix(q, k, v, ratio, gamma), D.ahla_loops(q, k, v, ratio, gamma)) < 1e-13


@pytest.mark.parametrize("n,d,dv", [(1, 3, 2), (17, 4, 3), (40, 6, 5)])
@pytest.mark.parametrize("ratio", [False, True])
def test_serial_equals_definition(n, d, dv, ratio):
    rng = np.random.default_rng(n + d)
    H, B = 2, 2
    q, k, v = rand_qkv(rng, B * H, n, d, dv, pos=ratio)
    gamma = np.array([0.9, 0.97])
    got = oracle.ahla(q, k, v, ratio=ratio, H=H, gamma=gamma)
    assert rel(got, D.ahla_batched(q, k, v, ratio, H, gamma)) < 1e-12


@pytest.mark.parametrize("gamma", [0.6, 0.9, 0.99])
def test_is_chained_decayed_linear_attention(gamma):
    rng = np.random.default_rng(32)
    q, k, v = (x[0].astype(np.float64) for x in rand_qkv(rng, 1, 50, 6, 4))
    want = _causal_la(q, k, _causal_la(q, k, v, gamma), gamma)
    assert rel(oracle.ahla(q[None], k[None], v[None], H=1, gamma=[gamma])[0], want) < 1e-12


@pytest.mark.parametrize("gamma", [0.5, 0.8, 0.95])
def test_unit_input_closed_form(gamma):
    # q = k = v = 1 (d = dv = 1): A = 1, o_t = sum_{j<=t} (t - j + 1) g^(t-j)
    #   = sum_{m=0}^{t} (m + 1) g^m = (1 - (t+2) g^(t+1) + (t+1) g^(t+2)) / (1 - g)^2
    n = 30
    one = np.ones((1, n, 1), np.float32)
    t = np.arange(n, dtype=np.float64)
    want = (1 - (t + 2) * gamma ** (t + 1) + (t + 1) * gamma ** (t + 2)) / (1 - gamma) ** 2
    np.testing.assert_allclose(oracle.ahla(one, one, one, H=1, gamma=[gamma])[0, :, 0], want,
                               rtol=1e-13)


def test_special_cases():
    rng = np.random.default_rng(33)
    q, k, v = rand_qkv(rng, 1, 25, 4, 3)
    # g = 1 is the undecayed operator, bit for bit (the same recurrence)
    assert np.array_equal(oracle.ahla(q, k, v, H=1, gamma=[1.0]), oracle.ahla(q, k, v))
    # g = 0 keeps only i = j = t: o_t = (q_t . k_t)^2 v_t
    qd, kd, vd = (x[0].astype(np.float64) for x in (q, k, v))
    want = ((qd * kd).sum(1) ** 2)[:, None] * vd
    assert rel(oracle.ahla(q, k, v, H=1, gamma=[0.0])[0], want) < 1e-13


def test_ratio_constant_values_and_causality():
    rng = np.random.default_rng(34)
    q, k, v = rand_qkv(rng, 1, 30, 4, 3, pos=True)
    c = np.ones_like(v) * np.array([0.25, -2.0, 7.0], np.float32)
    got = oracle.ahla(q, k, c, ratio=True, H=1, gamma=[0.9])
    assert rel(got, c) < 1e-14
    # moving token 20 leaves outputs 0..19 bit-identical
    o1 = oracle.ahla(q, k, v, H=1, gamma=[0.9])
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 20:] += 1.0
    k2[:, 20:] -= 0.5
    v2[:, 20:] *= 3.0
    o2 = oracle.ahla(q2, k2, v2, H=1, gamma=[0.9])
    assert np.array_equal(o1[:, :20], o2[:, :20]) and not np.array_equal(o1[:, 20:], o2[:, 20:])


@pytest.mark.parametrize("n", [1, 48, 67])
@pytest.mark.parametrize("chunk,seg", [(1, 1), (2, 3), (16, 1), (8, 5)])
@pytest.mark.parametrize("ratio", [False, True])
def test_scan_equals_serial(n, chunk, seg, ratio):
    rng = np.random.default_rng(n * 5 + chunk)
    q, k, v = rand_qkv(rng, 1, n, 5, 3, pos=ratio)
    g = 0.92
    o, st = oracle.ahla(q, k, v, ratio=ratio, want_state=True, H=1, gamma=[g])
    oc, stc = CS.ahla_scan_forward(q[0], k[0], v[0], chunk, seg, ratio, gamma=g)
    assert rel(oc, o[0]) < 1e-12
    for a, b in zip(stc, oracle.split_ahla_state(st[0], 5, 3)):
        assert rel(a, b) < 1e-12


def test_resume_and_scan_with_state_in():
    rng = np.random.default_rng(35)
    q, k, v = rand_qkv(rng, 1, 90, 4, 3)
    g = 0.95
    whole = oracle.ahla(q, k, v, H=1, gamma=[g])
    o1, st = oracle.ahla(q[:, :37], k[:, :37], v[:, :37], want_state=True, H=1, gamma=[g])
    o2 = oracle.ahla(q[:, 37:], k[:, 37:], v[:, 37:], state_in=st, H=1, gamma=[g])
    assert rel(np.concatenate([o1, o2], axis=1), whole) < 1e-13
    oc, _ = CS.ahla_scan_forward(q[0, 37:], k[0, 37:], v[0, 37:], 8, 2, gamma=g,
                                 state_in=oracle.split_ahla_state(st[0], 4, 3))
    assert rel(oc, whole[0, 37:]) < 1e-12


def test_combine_associative_with_identity():
    rng = np.random.default_rng(36)
    d, dv, g = 5, 3, 0.9

    def ra(l):
        return dict(P=rng.standard_normal((d, dv)), E=rng.standard_normal((d, dv)),
                    M=rng.standard_normal((d, d)), mK=rng.standard_normal(d),
                    nk=rng.standard_normal(d), l=l)
    a, b, c = ra(3), ra(7), ra(2)
    left = CS.ahla_combine(CS.ahla_combine(a, b, g), c, g)
    right = CS.ahla_combine(a, CS.ahla_combine(b, c, g), g)
    for key in ("P", "E", "M", "mK", "nk"):
        assert rel(left[key], right[key]) < 1e-14
    z = CS.ahla_zero(d, dv)
    for key in ("P", "E", "M", "mK", "nk"):
        assert rel(CS.ahla_combine(z, a, g)[key], a[key]) == 0.0
        assert rel(CS.ahla_combine(a, z, g)[key], a[key]) == 0.0


def test_pins_reject_plausible_mistakes():
    """The HLA-2 weight law g^((t-i)+(t-j)) applied to AHLA, decay on the
    inner or the outer factor only, and a decayed cross moment M_B in the
    combine each differ from the reading far beyond every tolerance above."""
    rng = np.random.default_rng(37)
    q, k, v = (x[0].astype(np.float64) for x in rand_qkv(rng, 1, 24, 4, 3))
    n, g = q.shape[0], 0.9
    good = oracle.ahla(q[None], k[None], v[None], H=1, gamma=[g])[0]
    L = np.tril(q @ k.T)
    Dg = D.decay_mask(n, g)
    t = np.arange(n)
    hla2_law = np.zeros((n, n))
    for tt in range(n):
        for j in range(tt + 1):
            hla2_law[tt, j] = sum(g ** ((tt - i) + (tt - j)) * L[tt, i] * L[i, j]
                                  for i in range(j, tt + 1))
    mistakes = {"hla2_weight_law": hla2_law @ v, "inner_only": (L @ (Dg * L)) @ v,
                "outer_only": ((Dg * L) @ L) @ v}
    for name, bad in mistakes.items():
        assert rel(bad, good) > 1e-2, name
    # a decayed M_B (instead of the plain sum) breaks scan == serial
    q32, k32, v32 = (x.astype(np.float32)[None] for x in (q, k, v))
    orig = CS.ahla_segment_summary

    def decayed_m(qq, kk, vv, chunk, gg=1.0):
        s = orig(qq, kk, vv, chunk, gg)
        w = gg ** (len(qq) - 1 - np.arange(len(qq)))
        s["M"] = (w[:, None] * kk).T @ qq
        return s
    CS.ahla_segment_summary = decayed_m
    try:
        oc, _ = CS.ahla_scan_forward(q, k, v, 4, 2, gamma=g)
    finally:
        CS.ahla_segment_summary = orig
    assert rel(oc, good) > 1e-3


@pytest.mark.parametrize("ratio", [False, True])
def test_backward_by_central_differences(ratio):
    """The oracle's AHLA gradient with a decay against central differences of
    its matrix definition, every entry."""
    rng = np.random.default_rng(38)
    q, k, v = (x[0].astype(np.float64) for x in rand_qkv(rng, 1, 9, 3, 2, pos=ratio))
    do = rng.standard_normal(v.shape)
    g = 0.8
    dq, dk, dv = BW.ahla_vjp(q, k, v, do, ratio, g)
    h = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            fp = (D.ahla_matrix(q, k, v, ratio, g) * do).sum()
            x[idx] = x0 - h
            fm = (D.ahla_matrix(q, k, v, ratio, g) * do).sum()
            x[idx] = x0
            num[idx] = (fp - fm) / (2 * h)
        assert rel(dx, num) < 1e-7
