"""Pins for the backward oracle (oracle/backward.py): its hand-applied chain
rule is checked against things that do not share it -- central finite
differences of the forward definition, PyTorch autograd (fp64, CPU) through
the masked matrix form, Euler's identity for the operators' homogeneity, and
causality of the gradient.

Forward operator: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
(gist.science/es/paper/2510.27258), "1. HLA de Segundo Orden" and "2. ...
(AHLA)"; training through the exact scan, "4. Entrenamiento Paralelo mediante
Escaneos Asociativos".
"""
import numpy as np
import pytest

from oracle import backward as BW
from oracle import definition as D


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def inputs(rng, n, d, dv, pos=False):
    if pos:
        q = rng.random((n, d)) + 0.1
        k = rng.random((n, d)) + 0.1
    else:
        q = rng.standard_normal((n, d))
        k = rng.standard_normal((n, d))
    return q, k, rng.standard_normal((n, dv)), rng.standard_normal((n, dv))


def forward(family, q, k, v, gamma, ratio):
    if family == "hla2":
        return D.hla2_matrix(q, k, v, gamma, ratio)
    return D.ahla_matrix(q, k, v, ratio)


def vjp(family, q, k, v, do, gamma, ratio):
    if family == "hla2":
        return BW.hla2_vjp(q, k, v, do, gamma, ratio)
    return BW.ahla_vjp(q, k, v, do, ratio)


CASES = [("hla2", 1.0, False), ("hla2", 0.8, False), ("hla2", 1.0, True), ("hla2", 0.7, True),
         ("ahla", 1.0, False), ("ahla", 1.0, True)]


@pytest.mark.parametrize("family,gamma,ratio", CASES)
def test_finite_differences(family, gamma, ratio):
    """Every entry of dq, dk, dv against a central difference of
    sum(do * o) through the brute-force forward definition."""
    rng = np.random.default_rng(11)
    n, d, dv = 7, 3, 2
    q, k, v, do = inputs(rng, n, d, dv, pos=ratio)
    got = vjp(family, q, k, v, do, gamma, ratio)
    h = 1e-6
    for which, x in enumerate((q, k, v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fp = np.sum(do * forward(family, *args_p, gamma, ratio))
            fm = np.sum(do * forward(family, *args_m, gamma, ratio))
            fd[idx] = (fp - fm) / (2 * h)
        assert rel(got[which], fd) < 1e-7, (which, rel(got[which], fd))


@pytest.mark.parametrize("family,gamma,ratio", CASES)
def test_autograd(family, gamma, ratio):
    """Against PyTorch autograd (fp64, CPU) through the explicit double sums of
    the definition, on a size where every token pair matters."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    n, d, dv = 24, 5, 4
    q, k, v, do = inputs(rng, n, d, dv, pos=ratio)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    A = tq @ tk.T
    t = torch.arange(n)
    rows = []
    for ti in range(n):
        num = torch.zeros(dv, dtype=torch.float64)
        den = torch.zeros((), dtype=torch.float64)
        if family == "hla2":
            # pairs i <= j <= t with weight g^((t-i)+(t-j)) A[t,i] A[j,i]
            for j in range(ti + 1):
                i = t[:j + 1]
                w = (gamma ** ((ti - i) + (ti - j)).double()) * A[ti, :j + 1] * A[j, :j + 1]
                num = num + w.sum() * tv[j]
                den = den + w.sum()
        else:
            # pairs j <= i <= t with weight A[t,i] A[i,j]
            for i in range(ti + 1):
                w = A[ti, i] * A[i, :i + 1]
                num = num + (w[:, None] * tv[:i + 1]).sum(0)
                den = den + w.sum()
        rows.append(num / den if ratio else num)
    o = torch.stack(rows)
    (o * torch.tensor(do)).sum().backward()
    got = vjp(family, q, k, v, do, gamma, ratio)
    for g, want in zip(got, (tq.grad, tk.grad, tv.grad)):
        assert rel(g, want.numpy()) < 1e-12


@pytest.mark.parametrize("family,gamma,ratio", CASES)
def test_euler_homogeneity(family, gamma, ratio):
    """o is homogeneous of degree 2 in q, 2 in k, 1 in v (ratio: 0, 0, 1), so
    <x, dx> = degree * <do, o> for each input x."""
    rng = np.random.default_rng(13)
    n, d, dv = 64, 8, 6
    q, k, v, do = inputs(rng, n, d, dv, pos=ratio)
    o = forward(family, q, k, v, gamma, ratio)
    dq, dk, dv_ = vjp(family, q, k, v, do, gamma, ratio)
    ref = float(np.sum(do * o))
    deg = (0, 0, 1) if ratio else (2, 2, 1)
    for x, g, p in zip((q, k, v), (dq, dk, dv_), deg):
        lhs = float(np.sum(x * g))
        scale = float(np.linalg.norm(x) * np.linalg.norm(g))
        assert abs(lhs - p * ref) <= 1e-10 * scale, (lhs, p * ref)


@pytest.mark.parametrize("family,gamma,ratio", CASES)
def test_gradient_causality(family, gamma, ratio):
    """With do zero from t0 on, nothing at or after t0 gets a gradient (the
    outputs before t0 never read those tokens), and moving those tokens
    leaves the gradient of the earlier ones bit-identical."""
    rng = np.random.default_rng(14)
    n, d, dv, t0 = 40, 4, 3, 23
    q, k, v, do = inputs(rng, n, d, dv, pos=ratio)
    do[t0:] = 0
    g1 = vjp(family, q, k, v, do, gamma, ratio)
    for g in g1:
        assert np.all(g[t0:] == 0)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[t0:] += 1.0
    k2[t0:] -= 0.5
    v2[t0:] *= 3.0
    g2 = vjp(family, q2, k2, v2, do, gamma, ratio)
    for a, b in zip(g1, g2):
        assert np.allclose(a[:t0], b[:t0], rtol=1e-12, atol=0)


def test_planted_mistakes_are_caught():
    """Each plausible slip in the chain rule -- the decay mask dropped from dN,
    the tril on dL dropped, dL taken transposed -- moves the gradient far
    outside the finite-difference agreement above."""
    rng = np.random.default_rng(15)
    n, d, dv, g = 9, 3, 2, 0.8
    q, k, v, do = inputs(rng, n, d, dv)
    dq, dk, dvv = BW.hla2_vjp(q, k, v, do, g)
    A = q @ k.T
    Dg = D.decay_mask(n, g)
    L, F = np.tril(A), Dg * A
    dM = do @ v.T
    variants = []
    dN = dM                                   # decay mask dropped
    variants.append((Dg * (dN @ L) + np.tril(dN.T @ F)) @ k)
    dN = Dg * dM
    variants.append((Dg * (dN @ L) + dN.T @ F) @ k)       # tril dropped
    variants.append((Dg * (dN @ L) + np.tril(F.T @ dN)) @ k)  # transposed
    for wrong in variants:
        assert rel(wrong, dq) > 1e-3


# ---------------------------------------------------------- decay gradient

def _fd_gamma(fwd, q, k, v, do, g, h=1e-6):
    return float(((fwd(g + h) - fwd(g - h)) * do).sum() / (2 * h))


@pytest.mark.parametrize("ratio", [False, True])
@pytest.mark.parametrize("gamma", [0.7, 0.95, 1.0])
def test_dgamma_finite_differences(gamma, ratio):
    """dL/dg by the chain rule against a central difference of the masked
    matrix definition (L = sum(dO * o)); at g = 1 the difference straddles
    the page's undecayed operator."""
    rng = np.random.default_rng(31 + int(100 * gamma) + ratio)
    n, d, dv = 23, 4, 3
    q, k, v, do = inputs(rng, n, d, dv, pos=ratio)
    fd = _fd_gamma(lambda g: D.hla2_matrix(q, k, v, g, ratio), q, k, v, do, gamma)
    got = BW.hla2_dgamma(q, k, v, do, gamma, ratio)
    assert abs(got - fd) <= 1e-6 * max(1.0, abs(fd))


def test_dgamma_loops_definition():
    """The same derivative against a central difference of the explicit
    double sum (a second, loop-based forward)."""
    rng = np.random.default_rng(37)
    n, d, dv, g = 7, 3, 2, 0.85
    q, k, v, do = inputs(rng, n, d, dv)
    fd = _fd_gamma(lambda gg: D.hla2_loops(q, k, v, gg), q, k, v, do, g)
    assert abs(BW.hla2_dgamma(q, k, v, do, g) - fd) <= 1e-6 * max(1.0, abs(fd))


def test_dgamma_special_cases():
    """One token: no pair (t, i) with i < t, so the decay never acts and
    dL/dg = 0.  Batched: per-(b, h) derivatives summed over b."""
    rng = np.random.default_rng(41)
    q, k, v, do = inputs(rng, 1, 4, 4)
    assert BW.hla2_dgamma(q, k, v, do, 0.9) == 0.0
    H, B, n, d = 2, 3, 6, 3
    x = [rng.standard_normal((B * H, n, d)) for _ in range(4)]
    gam = np.array([0.8, 0.95])
    got = BW.hla2_dgamma_batched(*x, H, gam)
    for h in range(H):
        want = sum(BW.hla2_dgamma(x[0][b * H + h], x[1][b * H + h], x[2][b * H + h],
                                  x[3][b * H + h], gam[h]) for b in range(B))
        assert got[h] == pytest.approx(want, rel=1e-12)


def test_dgamma_planted_mistakes_are_caught():
    """Dropping either mask's term, or using g^(t-i) in place of its
    derivative, moves dL/dg far from the finite difference."""
    rng = np.random.default_rng(43)
    n, d, dv, g = 11, 3, 2, 0.8
    q, k, v, do = inputs(rng, n, d, dv)
    fd = _fd_gamma(lambda gg: D.hla2_matrix(q, k, v, gg), q, k, v, do, g)
    A = q @ k.T
    Dg = D.decay_mask(n, g)
    lag = np.arange(n)[:, None] - np.arange(n)[None, :]
    dD = np.where(lag >= 1, lag * g ** np.maximum(lag - 1, 0), 0.0)
    L, F = np.tril(A), Dg * A
    N = F @ L.T
    dM = do @ v.T
    dF = (Dg * dM) @ L
    for wrong in ((dF * A * dD).sum(), (dM * N * dD).sum(),
                  (dF * A * Dg).sum() + (dM * N * Dg).sum()):
        assert abs(wrong - fd) > 1e-3 * abs(fd)
