"""Third-order masked HLA, fp64 -- TEST INFRASTRUCTURE ONLY.

Only the test suite may use this module (see ``oracle/__init__.py``); it
shares no code with the HIP library.

Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
(gist.science/es/paper/2510.27258), section "3. HLA de Tercer Orden": the
third-order operator is the matrix product A A^T A with A = Q K^T, made
strictly causal; its streaming form keeps the prefix moments S^K, S^Q, P^KV
plus cross-summaries (none of which the page prints).

Reading of the mask (the page gives none): every index of the product stays
at or before t, with each factor lower-triangular as in the second-order
case (o = tril(L L^T) V there):

    o = tril(L L^T) L V,   L = tril(Q K^T) (diagonal kept), i.e.
    o_t = sum_{m<=t} sum_{i<=m} sum_{j<=m} A[t,i] A[m,i] A[m,j] v_j .

Without the masks this is Q (K^T K)(Q^T Q)(K^T V) = q_t^T S^K S^Q P^KV, the
three moments the page names.  The other placements of the mask (no inner
tril, or L tril(L^T L)) sum over m > t, i.e. over future tokens.

Three forms are written out: explicit loops (tiny n), the matrix product,
and a serial recurrence with an O(d^2 + d dv) state per token
(P = sum k v^T gives y_m = P^T q_m; then S = sum k k^T, z = S q, W = sum z y^T,
o = q^T W).

Decay ("Contribuciones Clave", item 2, names masked operators with and
without exponential decay; the same reading as for second order): every
streaming moment decays by g per token.  The unmasked product is then
q_t^T S^K_t S^Q_t P^KV_t with each moment decayed to t, so the term
(i, m, j) carries g^((t-i)+(t-m)+(t-j)); in the recurrence P <- g P + k v^T,
S <- g S + k k^T and W <- g^3 W + z y^T (z_m and y_m are already decayed to
m, and the pair's remaining weight to t is g^(3(t-m))).

Ratio form (as for second order: the numerator over the same operator with
v == 1): den_t = sum_{m,i,j} g^(...) A[t,i] A[m,i] A[m,j], o_t = num_t / den_t.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def hla3_loops(q, k, v, gamma: float = 1.0, ratio: bool = False):
    """Direct triple sum for one head; q, k: [n, d], v: [n, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, dv = v.shape
    o = np.zeros((n, dv))
    for t in range(n):
        den = 0.0
        for m in range(t + 1):
            for i in range(m + 1):
                a = float(q[t] @ k[i]) * float(q[m] @ k[i])
                for j in range(m + 1):
                    w = gamma ** ((t - i) + (t - m) + (t - j)) * a * float(q[m] @ k[j])
                    o[t] += w * v[j]
                    den += w
        if ratio:
            o[t] /= den
    return o


def _decay(n, g):
    t = np.arange(n)
    lag = t[:, None] - t[None, :]
    return np.where(lag >= 0, float(g) ** np.maximum(lag, 0), 0.0)


def hla3_matrix(q, k, v, gamma: float = 1.0, ratio: bool = False):
    """Matrix form for one head (materialises n x n):
    o = (D_{g^3} * (L F^T)) F V with F = D_g * L, L = tril(Q K^T)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    A = q @ k.T
    F = _decay(n, gamma) * A
    M = _decay(n, gamma ** 3) * (A @ F.T)
    num = M @ (F @ v)
    if ratio:
        return num / (M @ F.sum(axis=1))[:, None]
    return num


def hla3_serial(q, k, v, gamma: float = 1.0, ratio: bool = False):
    """Serial recurrence for one head, fp64: per token t
        P <- g P + k_t v_t^T;  y_t = P^T q_t;  S <- g S + k_t k_t^T;
        z_t = S q_t;  W <- g^3 W + z_t y_t^T;  o_t = W^T q_t
    (ratio: the same recurrence on v == 1 alongside, o_t / den_t)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[1]
    g, g3 = float(gamma), float(gamma) ** 3
    P = np.zeros((d, dv))
    S = np.zeros((d, d))
    W = np.zeros((d, dv))
    p1 = np.zeros(d)
    w1 = np.zeros(d)
    o = np.empty((n, dv))
    for t in range(n):
        P = g * P + np.outer(k[t], v[t])
        y = P.T @ q[t]
        S = g * S + np.outer(k[t], k[t])
        z = S @ q[t]
        W = g3 * W + np.outer(z, y)
        o[t] = W.T @ q[t]
        if ratio:
            p1 = g * p1 + k[t]
            w1 = g3 * w1 + z * float(p1 @ q[t])
            o[t] /= float(w1 @ q[t])
    return o


def hla3_batched(q, k, v, heads=None, H: int = 1, gamma=None, ratio: bool = False):
    """Matrix form over [BH, n, *] arrays (or the listed head indices); gamma
    is None or a length-H array indexed by h = bh % H."""
    bhs = range(q.shape[0]) if heads is None else heads
    return np.stack([hla3_matrix(q[bh], k[bh], v[bh],
                                 1.0 if gamma is None else float(gamma[bh % H]), ratio)
                     for bh in bhs])


def hla3_serial_state(q, k, v, gamma: float = 1.0, ratio: bool = False, state=None):
    """The serial recurrence from and to an explicit state, for one head:
    state = (P, S, W) and, for the ratio form, also (p1, w1), the same
    moments of the v == 1 chain.  Returns (o, state)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[1]
    g, g3 = float(gamma), float(gamma) ** 3
    if state is None:
        state = (np.zeros((d, dv)), np.zeros((d, d)), np.zeros((d, dv))) + \
            ((np.zeros(d), np.zeros(d)) if ratio else ())
    P, S, W = (np.array(x, np.float64) for x in state[:3])
    p1, w1 = (np.array(x, np.float64) for x in state[3:5]) if ratio else (None, None)
    o = np.empty((n, dv))
    for t in range(n):
        P = g * P + np.outer(k[t], v[t])
        y = P.T @ q[t]
        S = g * S + np.outer(k[t], k[t])
        z = S @ q[t]
        W = g3 * W + np.outer(z, y)
        o[t] = W.T @ q[t]
        if ratio:
            p1 = g * p1 + k[t]
            w1 = g3 * w1 + z * float(p1 @ q[t])
            o[t] /= float(w1 @ q[t])
    return o, ((P, S, W) + ((p1, w1) if ratio else ()))


def hla3_vjp(q, k, v, do, gamma: float = 1.0, ratio: bool = False):
    """(dq, dk, dv) for one head: the chain rule through the matrix form
    o = P Y, P = D_{g^3} * (A F^T), Y = F V, F = D_g * A (ratio: num / den
    with den = P (F 1))."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    D1, D3 = _decay(n, gamma), _decay(n, gamma ** 3)
    A = q @ k.T
    F = D1 * A
    P = D3 * (A @ F.T)
    Y = F @ v
    if ratio:
        y1 = F.sum(axis=1)
        den = P @ y1
        o = (P @ Y) / den[:, None]
        G = do / den[:, None]
        e = -(do * o).sum(axis=1) / den          # upstream of den
        dP = G @ Y.T + np.outer(e, y1)
        dY = P.T @ G
        dy1 = P.T @ e
    else:
        dP = do @ Y.T
        dY = P.T @ do
        dy1 = None
    dv = F.T @ dY
    dAF = D3 * dP                                 # gradient of A F^T
    dA = dAF @ F
    dF = dAF.T @ A + dY @ v.T
    if ratio:
        dF += np.outer(dy1, np.ones(n))
    dA += D1 * dF
    return dA @ k, dA.T @ q, dv


def hla3_vjp_batched(q, k, v, do, H: int = 1, gamma=None, ratio: bool = False, heads=None):
    bhs = range(q.shape[0]) if heads is None else heads
    res = [hla3_vjp(q[bh], k[bh], v[bh], do[bh],
                    1.0 if gamma is None else float(gamma[bh % H]), ratio) for bh in bhs]
    return tuple(np.stack([r[i] for r in res]) for i in range(3))
