"""Pins for the oracle: every check here compares it with something other than
itself -- the explicit double sums of the masked definition, hand-worked
values, closed forms, the chained causal-linear-attention reduction, and
invariants the pages state (causality, exact scan == serial).

Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
(gist.science/es/paper/2510.27258): "1. HLA de Segundo Orden",
"2. ... (AHLA)", "4. Entrenamiento Paralelo mediante Escaneos Asociativos",
"Resultados y Afirmaciones" (causality, exactness).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunk_scan as CS
from oracle import definition as D

GOLD = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rand_qkv(rng, BH, n, d, dv, pos=False):
    if pos:
        q = rng.random((BH, n, d)) / np.sqrt(d)
        k = rng.random((BH, n, d)) / np.sqrt(d)
    else:
        q = rng.standard_normal((BH, n, d)) / np.sqrt(d)
        k = rng.standard_normal((BH, n, d)) / np.sqrt(d)
    v = rng.standard_normal((BH, n, dv))
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_lib):
    return oracle_lib


# ---------------------------------------------------------------- golden values

def test_golden_ones_closed_form():
    g = json.load(open(GOLD))["ones_d1"]
    n = g["n"]
    one = np.ones((1, n, 1), np.float32)
    np.testing.assert_allclose(oracle.hla2(one, one, one)[0, :, 0], g["hla2"], rtol=0, atol=0)
    np.testing.assert_allclose(oracle.ahla(one, one, one)[0, :, 0], g["ahla"], rtol=0, atol=0)
    # and for long sequences the formula (t+1)(t+2)/2
    n = 300
    one = np.ones((1, n, 1), np.float32)
    t = np.arange(n)
    np.testing.assert_allclose(oracle.hla2(one, one, one)[0, :, 0], (t + 1) * (t + 2) / 2, rtol=1e-14)
    np.testing.assert_allclose(oracle.ahla(one, one, one)[0, :, 0], (t + 1) * (t + 2) / 2, rtol=1e-14)


def test_golden_decay_half():
    g = json.load(open(GOLD))["ones_d1_decay_half"]
    n = len(g["hla2"])
    one = np.ones((1, n, 1), np.float32)
    o = oracle.hla2(one, one, one, H=1, gamma=[g["gamma"]])[0, :, 0]
    np.testing.assert_allclose(o, g["hla2"], rtol=1e-15)


@pytest.mark.parametrize("gamma", [0.5, 0.9, 0.999])
def test_decay_geometric_double_sum(gamma):
    # closed form of sum_{j<=t} sum_{i<=j} g^((t-i)+(t-j)) for unit inputs:
    # with a = t - j, b = j - i: g^(2a+b), a in [0,t], b in [0, t-a]
    n = 64
    one = np.ones((1, n, 1), np.float32)
    o = oracle.hla2(one, one, one, H=1, gamma=[gamma])[0, :, 0]
    want = []
    for t in range(n):
        s = 0.0
        for a in range(t + 1):
            s += gamma ** (2 * a) * (1 - gamma ** (t - a + 1)) / (1 - gamma)
        want.append(s)
    np.testing.assert_allclose(o, want, rtol=1e-12)


def test_golden_single_and_two_tokens():
    gold = json.load(open(GOLD))
    for c in gold["single_token"]["cases"]:
        q = np.array(c["q"], np.float32)[None, None]
        k = np.array(c["k"], np.float32)[None, None]
        v = np.array(c["v"], np.float32)[None, None]
        np.testing.assert_allclose(oracle.hla2(q, k, v)[0, 0], c["o"], rtol=1e-15)
        np.testing.assert_allclose(oracle.ahla(q, k, v)[0, 0], c["o"], rtol=1e-15)
    g2 = gold["two_tokens"]
    q = np.array(g2["q"], np.float32)[None, :, None]
    k = np.array(g2["k"], np.float32)[None, :, None]
    v = np.array(g2["v"], np.float32)[None, :, None]
    np.testing.assert_allclose(oracle.hla2(q, k, v)[0, :, 0], g2["hla2"], rtol=1e-15)
    np.testing.assert_allclose(oracle.ahla(q, k, v)[0, :, 0], g2["ahla"], rtol=1e-15)


# ------------------------------------------------------------ rank-one closed forms

def test_constant_key_closed_form():
    # k_i = k for all i, a_t = q_t . k:
    #   HLA-2 o_t = a_t sum_{j<=t} (j+1) a_j v_j     (j+1 keys at or before j)
    #   AHLA  o_t = a_t sum_{i<=t} a_i sum_{j<=i} v_j
    rng = np.random.default_rng(5)
    n, d, dv = 40, 6, 3
    q = rng.standard_normal((1, n, d)).astype(np.float32)
    kk = rng.standard_normal(d).astype(np.float32)
    k = np.broadcast_to(kk, (1, n, d)).copy()
    v = rng.standard_normal((1, n, dv)).astype(np.float32)
    a = q[0].astype(np.float64) @ kk.astype(np.float64)
    vv = v[0].astype(np.float64)
    want_h = np.array([a[t] * sum((j + 1) * a[j] * vv[j] for j in range(t + 1)) for t in range(n)])
    cv = np.cumsum(vv, axis=0)
    want_a = np.array([a[t] * sum(a[i] * cv[i] for i in range(t + 1)) for t in range(n)])
    assert rel(oracle.hla2(q, k, v)[0], want_h) < 1e-13
    assert rel(oracle.ahla(q, k, v)[0], want_a) < 1e-13


def test_constant_query_closed_form():
    # q_t = q for all t, b_i = q . k_i:
    #   HLA-2 o_t = sum_{j<=t} (sum_{i<=j} b_i^2) v_j
    #   AHLA  o_t = sum_{i<=t} b_i sum_{j<=i} b_j v_j
    rng = np.random.default_rng(6)
    n, d, dv = 40, 5, 2
    qq = rng.standard_normal(d).astype(np.float32)
    q = np.broadcast_to(qq, (1, n, d)).copy()
    k = rng.standard_normal((1, n, d)).astype(np.float32)
    v = rng.standard_normal((1, n, dv)).astype(np.float32)
    b = k[0].astype(np.float64) @ qq.astype(np.float64)
    vv = v[0].astype(np.float64)
    cb2 = np.cumsum(b * b)
    want_h = np.cumsum(cb2[:, None] * vv, axis=0)
    inner = np.cumsum(b[:, None] * vv, axis=0)
    want_a = np.cumsum(b[:, None] * inner, axis=0)
    assert rel(oracle.hla2(q, k, v)[0], want_h) < 1e-13
    assert rel(oracle.ahla(q, k, v)[0], want_a) < 1e-13


# ------------------------------------------------------ definition: loops == matrix

@pytest.mark.parametrize("gamma,ratio", [(1.0, False), (0.8, False), (1.0, True), (0.9, True)])
def test_matrix_form_equals_double_sum(gamma, ratio):
    rng = np.random.default_rng(1)
    q, k, v = rand_qkv(rng, 1, 11, 3, 2, pos=ratio)
    assert rel(D.hla2_matrix(q[0], k[0], v[0], gamma, ratio),
               D.hla2_loops(q[0], k[0], v[0], gamma, ratio)) < 1e-13


@pytest.mark.parametrize("ratio", [False, True])
def test_ahla_matrix_form_equals_double_sum(ratio):
    rng = np.random.default_rng(2)
    q, k, v = rand_qkv(rng, 1, 11, 3, 2, pos=ratio)
    assert rel(D.ahla_matrix(q[0], k[0], v[0], ratio), D.ahla_loops(q[0], k[0], v[0], ratio)) < 1e-13


# ------------------------------------------------- serial oracle == brute force

@pytest.mark.parametrize("n,d,dv", [(1, 1, 1), (2, 3, 1), (17, 4, 5), (64, 8, 8), (33, 16, 4)])
@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("ratio", [False, True])
def test_hla2_serial_equals_definition(n, d, dv, decay, ratio):
    rng = np.random.default_rng(n * 100 + d)
    BH, H = 4, 2
    q, k, v = rand_qkv(rng, BH, n, d, dv, pos=ratio)
    gamma = np.array([0.93, 0.71]) if decay else None
    o = oracle.hla2(q, k, v, H=H, gamma=gamma, ratio=ratio)
    ref = D.hla2_batched(q, k, v, H, gamma, ratio)
    assert rel(o, ref) < 1e-12


@pytest.mark.parametrize("n,d,dv", [(1, 1, 1), (2, 3, 1), (17, 4, 5), (64, 8, 8)])
@pytest.mark.parametrize("ratio", [False, True])
def test_ahla_serial_equals_definition(n, d, dv, ratio):
    rng = np.random.default_rng(n * 7 + d)
    q, k, v = rand_qkv(rng, 3, n, d, dv, pos=ratio)
    assert rel(oracle.ahla(q, k, v, ratio=ratio), D.ahla_batched(q, k, v, ratio)) < 1e-12


def test_small_fp32_workload_whole_by_brute_force():
    # the whole 256-token, d = 16 fp32 workload is small enough for n x n
    from causal_streaming_scans_amd.inputs import workload_inputs
    x = workload_inputs("small_f32")
    o = oracle.hla2(x["q"], x["k"], x["v"])
    assert rel(o, D.hla2_batched(x["q"], x["k"], x["v"], 1)) < 1e-12


# -------------------------------------- chained causal linear attention reduction

def _causal_la(q, k, v, g=1.0):
    """Causal linear attention by its own recurrence: M <- g M + k v^T,
    out_t = M^T q_t (textbook form, written independently of the HLA code)."""
    n, d = q.shape
    M = np.zeros((d, v.shape[1]))
    out = np.zeros((n, v.shape[1]))
    for t in range(n):
        M = g * M + np.outer(k[t], v[t])
        out[t] = q[t] @ M
    return out


@pytest.mark.parametrize("gamma", [1.0, 0.85])
def test_hla2_is_chained_linear_attention(gamma):
    # HLA-2 = LA_{g^2}(Q, LA_g(Q, K, K), V): the second-order operator is
    # causal linear attention whose keys are the first-order read-outs S_t q_t.
    rng = np.random.default_rng(11)
    q, k, v = (x[0].astype(np.float64) for x in rand_qkv(rng, 1, 50, 6, 4))
    z = _causal_la(q, k, k, gamma)
    want = _causal_la(q, z, v, gamma * gamma)
    got = oracle.hla2(q[None], k[None], v[None], H=1, gamma=[gamma])[0]
    assert rel(got, want) < 1e-12


def test_ahla_is_chained_linear_attention():
    # AHLA = LA(Q, K, LA(Q, K, V))
    rng = np.random.default_rng(12)
    q, k, v = (x[0].astype(np.float64) for x in rand_qkv(rng, 1, 50, 6, 4))
    want = _causal_la(q, k, _causal_la(q, k, v))
    assert rel(oracle.ahla(q[None], k[None], v[None])[0], want) < 1e-12


# ------------------------------------------------------------------- invariants

def test_ratio_constant_values_returns_the_value():
    rng = np.random.default_rng(3)
    BH, n, d, dv = 3, 70, 8, 5
    q, k, _ = rand_qkv(rng, BH, n, d, dv, pos=True)
    c = rng.standard_normal((BH, 1, dv)).astype(np.float32)
    v = np.broadcast_to(c, (BH, n, dv)).copy()
    for o in (oracle.hla2(q, k, v, ratio=True),
              oracle.hla2(q, k, v, H=3, gamma=[0.9, 0.95, 0.99], ratio=True),
              oracle.ahla(q, k, v, ratio=True)):
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-12, atol=1e-12)


def test_homogeneity_and_ratio_scale_invariance():
    rng = np.random.default_rng(4)
    q, k, v = rand_qkv(rng, 2, 30, 4, 3, pos=True)
    al, be = 2.0, 0.5  # exact in fp32
    o = oracle.hla2(q, k, v)
    assert rel(oracle.hla2(al * q, be * k, v), al ** 2 * be ** 2 * o) < 1e-14
    oa = oracle.ahla(q, k, v)
    assert rel(oracle.ahla(al * q, be * k, v), al ** 2 * be ** 2 * oa) < 1e-14
    r = oracle.hla2(q, k, v, ratio=True)
    assert rel(oracle.hla2(al * q, be * k, v, ratio=True), r) < 1e-14


@pytest.mark.parametrize("which", ["hla2", "hla2_decay", "ahla"])
def test_causality_bit_exact(which):
    # the output at t depends only on tokens j <= t: perturbing the future
    # leaves the earlier outputs bit-identical in the serial oracle
    rng = np.random.default_rng(8)
    q, k, v = rand_qkv(rng, 2, 40, 5, 3)
    t0 = 23
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, t0 + 1:] += 1.0
    k2[:, t0 + 1:] -= 0.5
    v2[:, t0 + 1:] *= 3.0
    f = {"hla2": lambda a, b, c: oracle.hla2(a, b, c),
         "hla2_decay": lambda a, b, c: oracle.hla2(a, b, c, H=2, gamma=[0.9, 0.97]),
         "ahla": lambda a, b, c: oracle.ahla(a, b, c)}[which]
    o1, o2 = f(q, k, v), f(q2, k2, v2)
    assert np.array_equal(o1[:, :t0 + 1], o2[:, :t0 + 1])
    assert not np.allclose(o1[:, t0 + 1:], o2[:, t0 + 1:])


def test_hla2_state_out_matches_direct_sums():
    # S = sum g^(n-1-i) k k^T ; W = sum_j g^(2(n-1-j)) z_j v_j^T ; u = sum g^(2(n-1-j)) z_j
    # with z_j = sum_{i<=j} g^(j-i) k_i (k_i . q_j), all evaluated directly
    rng = np.random.default_rng(9)
    n, d, dv, g = 25, 4, 3, 0.9
    q, k, v = rand_qkv(rng, 1, n, d, dv)
    _, st = oracle.hla2(q, k, v, H=1, gamma=[g], want_state=True)
    S, W, u = oracle.split_hla2_state(st[0], d, dv)
    q64, k64, v64 = (x[0].astype(np.float64) for x in (q, k, v))
    S_ref = sum(g ** (n - 1 - i) * np.outer(k64[i], k64[i]) for i in range(n))
    z = np.array([sum(g ** (j - i) * k64[i] * (k64[i] @ q64[j]) for i in range(j + 1))
                  for j in range(n)])
    W_ref = sum(g ** (2 * (n - 1 - j)) * np.outer(z[j], v64[j]) for j in range(n))
    u_ref = sum(g ** (2 * (n - 1 - j)) * z[j] for j in range(n))
    assert rel(S, S_ref) < 1e-13 and rel(W, W_ref) < 1e-13 and rel(u, u_ref) < 1e-13


def test_ahla_state_out_matches_direct_sums():
    rng = np.random.default_rng(10)
    n, d, dv = 25, 4, 3
    q, k, v = rand_qkv(rng, 1, n, d, dv)
    _, st = oracle.ahla(q, k, v, want_state=True)
    P, E, mK, nk = oracle.split_ahla_state(st[0], d, dv)
    q64, k64, v64 = (x[0].astype(np.float64) for x in (q, k, v))
    A = q64 @ k64.T
    y = np.array([sum(A[i, j] * v64[j] for j in range(i + 1)) for i in range(n)])
    y1 = np.array([A[i, :i + 1].sum() for i in range(n)])
    assert rel(P, k64.T @ v64) < 1e-13
    assert rel(E, k64.T @ y) < 1e-13
    assert rel(mK, k64.sum(0)) < 1e-13
    assert rel(nk, k64.T @ y1) < 1e-13


@pytest.mark.parametrize("variant", ["hla2", "hla2_ratio_decay", "ahla", "ahla_ratio"])
def test_forward_then_resume_equals_whole(variant):
    # the streaming state is the checkpoint: forward(n) -> state -> forward(m)
    # from that state equals forward(n + m)
    rng = np.random.default_rng(13)
    BH, n1, n2, d, dv = 3, 29, 18, 6, 4
    ratio = "ratio" in variant
    q, k, v = rand_qkv(rng, BH, n1 + n2, d, dv, pos=ratio)
    if variant.startswith("hla2"):
        kw = dict(H=3, gamma=[0.9, 0.95, 0.99]) if "decay" in variant else {}
        whole = oracle.hla2(q, k, v, ratio=ratio, **kw)
        o1, st = oracle.hla2(q[:, :n1], k[:, :n1], v[:, :n1], ratio=ratio, want_state=True, **kw)
        o2 = oracle.hla2(q[:, n1:], k[:, n1:], v[:, n1:], ratio=ratio, state_in=st, **kw)
    else:
        whole = oracle.ahla(q, k, v, ratio=ratio)
        o1, st = oracle.ahla(q[:, :n1], k[:, :n1], v[:, :n1], ratio=ratio, want_state=True)
        o2 = oracle.ahla(q[:, n1:], k[:, n1:], v[:, n1:], ratio=ratio, state_in=st)
    assert rel(np.concatenate([o1, o2], axis=1), whole) < 1e-12


# --------------------------------------------------------- scan == serial (exact)

@pytest.mark.parametrize("n", [1, 5, 48, 67])
@pytest.mark.parametrize("chunk,seg", [(1, 1), (2, 3), (3, 1), (16, 1), (16, 2), (8, 5), (64, 1)])
@pytest.mark.parametrize("gamma,ratio", [(1.0, False), (0.9, True)])
def test_hla2_scan_equals_serial(n, chunk, seg, gamma, ratio):
    rng = np.random.default_rng(n + chunk + seg)
    q, k, v = rand_qkv(rng, 1, n, 5, 3, pos=ratio)
    o, st = oracle.hla2(q, k, v, H=1, gamma=[gamma], ratio=ratio, want_state=True)
    oc, (S, W, u) = CS.hla2_scan_forward(q[0], k[0], v[0], chunk, seg, gamma, ratio)
    assert rel(oc, o[0]) < 1e-12
    S_o, W_o, u_o = oracle.split_hla2_state(st[0], 5, 3)
    assert rel(S, S_o) < 1e-12 and rel(W, W_o) < 1e-12 and rel(u, u_o) < 1e-12


@pytest.mark.parametrize("n", [1, 48, 67])
@pytest.mark.parametrize("chunk,seg", [(1, 1), (2, 3), (16, 1), (8, 5)])
@pytest.mark.parametrize("ratio", [False, True])
def test_ahla_scan_equals_serial(n, chunk, seg, ratio):
    rng = np.random.default_rng(n * 3 + chunk)
    q, k, v = rand_qkv(rng, 1, n, 5, 3, pos=ratio)
    o, st = oracle.ahla(q, k, v, ratio=ratio, want_state=True)
    oc, stc = CS.ahla_scan_forward(q[0], k[0], v[0], chunk, seg, ratio)
    assert rel(oc, o[0]) < 1e-12
    for a, b in zip(stc, oracle.split_ahla_state(st[0], 5, 3)):
        assert rel(a, b) < 1e-12


def test_scan_with_state_in_equals_serial():
    rng = np.random.default_rng(21)
    q, k, v = rand_qkv(rng, 1, 90, 4, 3)
    whole = oracle.hla2(q, k, v, H=1, gamma=[0.95])
    _, st = oracle.hla2(q[:, :37], k[:, :37], v[:, :37], H=1, gamma=[0.95], want_state=True)
    oc, _ = CS.hla2_scan_forward(q[0, 37:], k[0, 37:], v[0, 37:], 8, 2, 0.95,
                                 state_in=oracle.split_hla2_state(st[0], 4, 3))
    assert rel(oc, whole[0, 37:]) < 1e-12
    whole = oracle.ahla(q, k, v)
    _, st = oracle.ahla(q[:, :37], k[:, :37], v[:, :37], want_state=True)
    oc, _ = CS.ahla_scan_forward(q[0, 37:], k[0, 37:], v[0, 37:], 8, 2,
                                 state_in=oracle.split_ahla_state(st[0], 4, 3))
    assert rel(oc, whole[0, 37:]) < 1e-12


def _rand_hla2_summary(rng, d, dv, l):
    return dict(S=rng.standard_normal((d, d)), C=rng.standard_normal((d, dv)),
                m=rng.standard_normal(d), W=rng.standard_normal((d, dv)),
                u=rng.standard_normal(d), l=l)


def test_semidirect_combine_is_associative_with_identity():
    rng = np.random.default_rng(14)
    d, dv, g = 5, 3, 0.93
    a, b, c = (_rand_hla2_summary(rng, d, dv, l) for l in (3, 7, 2))
    left = CS.hla2_combine(CS.hla2_combine(a, b, g), c, g)
    right = CS.hla2_combine(a, CS.hla2_combine(b, c, g), g)
    for key in "SCmWu":
        assert rel(left[key], right[key]) < 1e-14
    z = CS.hla2_zero(d, dv)
    for key in "SCmWu":
        assert rel(CS.hla2_combine(z, a, g)[key], a[key]) == 0.0
        assert rel(CS.hla2_combine(a, z, g)[key], a[key]) == 0.0
    # and it is not commutative (the cross term is ordered)
    assert rel(CS.hla2_combine(a, b, g)["W"], CS.hla2_combine(b, a, g)["W"]) > 1e-3

    def ra():
        return dict(P=rng.standard_normal((d, dv)), E=rng.standard_normal((d, dv)),
                    M=rng.standard_normal((d, d)), mK=rng.standard_normal(d),
                    nk=rng.standard_normal(d))
    a, b, c = ra(), ra(), ra()
    left = CS.ahla_combine(CS.ahla_combine(a, b), c)
    right = CS.ahla_combine(a, CS.ahla_combine(b, c))
    for key in ("P", "E", "M", "mK", "nk"):
        assert rel(left[key], right[key]) < 1e-14


def test_blelloch_exclusive_matches_sequential_fold():
    # the tree scan with a non-commutative operator equals the left fold
    words = [chr(ord("a") + i) for i in range(11)]
    ex = CS.blelloch_exclusive(words, lambda x, y: x + y, lambda: "")
    assert ex == ["".join(words[:i]) for i in range(len(words))]


# ------------------------------------------- the pins catch plausible mistakes

def test_pins_reject_plausible_mistakes():
    """Each plausible slip in the oracle's algebra (strict instead of inclusive
    mask, transposed score, missing cross-summary, single-sided decay, AHLA
    operands swapped) changes the result far beyond the tolerances used above,
    so the brute-force and closed-form pins would fail on it."""
    rng = np.random.default_rng(15)
    q, k, v = (x[0].astype(np.float64) for x in rand_qkv(rng, 1, 24, 4, 3))
    n = q.shape[0]
    good = oracle.hla2(q[None], k[None], v[None], H=1, gamma=[0.9])[0]
    A = q @ k.T
    Dg = D.decay_mask(n, 0.9)
    mistakes = {
        "strict_mask": (Dg * ((Dg * np.tril(A, -1)) @ np.tril(A, -1).T)) @ v,
        "transposed_score": (Dg * ((Dg * A.T) @ np.tril(A.T).T)) @ v,
        "no_cross_summary": np.stack([q[t] @ (sum(0.9 ** (t - i) * np.outer(k[i], k[i]) for i in range(t + 1))
                                              @ sum(0.9 ** (t - j) * np.outer(q[j], v[j]) for j in range(t + 1)))
                                      for t in range(n)]),
        "one_sided_decay": (np.tril(np.ones((n, n))) * ((Dg * A) @ np.tril(A).T)) @ v,
    }
    for name, bad in mistakes.items():
        assert rel(bad, good) > 1e-2, name
    ga = oracle.ahla(q[None], k[None], v[None])[0]
    L = np.tril(A)
    assert rel((L @ L.T) @ v, ga) > 1e-2
    assert rel(np.tril(L.T @ L) @ v, ga) > 1e-2
