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
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def hla3_loops(q, k, v):
    """Direct triple sum for one head; q, k: [n, d], v: [n, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, dv = v.shape
    o = np.zeros((n, dv))
    for t in range(n):
        for m in range(t + 1):
            for i in range(m + 1):
                a = float(q[t] @ k[i]) * float(q[m] @ k[i])
                for j in range(m + 1):
                    o[t] += a * float(q[m] @ k[j]) * v[j]
    return o


def hla3_matrix(q, k, v):
    """Matrix form for one head (materialises n x n)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    L = np.tril(q @ k.T)
    return np.tril(L @ L.T) @ (L @ v)


def hla3_serial(q, k, v):
    """Serial recurrence for one head, fp64: per token t
        P += k_t v_t^T;  y_t = P^T q_t;  S += k_t k_t^T;  z_t = S q_t;
        W += z_t y_t^T;  o_t = W^T q_t ."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[1]
    P = np.zeros((d, dv))
    S = np.zeros((d, d))
    W = np.zeros((d, dv))
    o = np.empty((n, dv))
    for t in range(n):
        P += np.outer(k[t], v[t])
        y = P.T @ q[t]
        S += np.outer(k[t], k[t])
        z = S @ q[t]
        W += np.outer(z, y)
        o[t] = W.T @ q[t]
    return o


def hla3_batched(q, k, v, heads=None):
    """Matrix form over [BH, n, *] arrays (or the listed head indices)."""
    bhs = range(q.shape[0]) if heads is None else heads
    return np.stack([hla3_matrix(q[bh], k[bh], v[bh]) for bh in bhs])
