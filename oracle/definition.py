"""Brute-force evaluation of the masked HLA-2 / AHLA operators, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

These functions materialise the n x n score matrix and are meant for small n.
They are the plain definitions the streaming summaries of
"Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
(gist.science/es/paper/2510.27258) reach exactly:

* section "1. HLA de Segundo Orden": strictly causal second-order operator
  built from A = Q K^T; causality per "Resultados y Afirmaciones" (the output at
  t depends only on tokens j <= t, the diagonal included);
* section "2. ... (AHLA)": the asymmetric operator Q (K^T Q)(K^T V), masked;
* "Contribuciones Clave" item 2: the masked operators with exponential decay.

Notation: A[t, i] = q_t . k_i ; L = tril(A) (inclusive);
D_g[t, i] = g^(t - i) if i <= t else 0.

    HLA-2          o_t = sum_{j<=t} sum_{i<=j} g^((t-i)+(t-j)) A[t,i] A[j,i] v_j
                   i.e.  o = (D_g * ((D_g * A) L^T)) V
    ratio HLA-2    the same with v == 1 as denominator
    AHLA           o_t = sum_{i<=t} sum_{j<=i} g^(t-j) A[t,i] A[i,j] v_j
                   i.e.  o = ((D_g * L)(D_g * L)) V = (D_g * (L L)) V
    ratio AHLA     the same with v == 1 as denominator

Decay (both families) is the reading in which every streaming summary decays
by g per token; g = 1 is the undecayed operator.

Two forms are given: explicit loops (``*_loops``, tiny inputs only) and the
equivalent matrix expressions (``hla2_matrix``, ``ahla_matrix``).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def hla2_loops(q, k, v, gamma: float = 1.0, ratio: bool = False):
    """Direct double sum for one head; q, k: [n, d], v: [n, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, dv = v.shape
    o = np.zeros((n, dv))
    for t in range(n):
        num = np.zeros(dv)
        den = 0.0
        for j in range(t + 1):
            for i in range(j + 1):
                w = gamma ** ((t - i) + (t - j)) * float(q[t] @ k[i]) * float(q[j] @ k[i])
                num += w * v[j]
                den += w
        o[t] = num / den if ratio else num
    return o


def ahla_loops(q, k, v, ratio: bool = False, gamma: float = 1.0):
    """Direct double sum for one head; q, k: [n, d], v: [n, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, dv = v.shape
    o = np.zeros((n, dv))
    for t in range(n):
        num = np.zeros(dv)
        den = 0.0
        for i in range(t + 1):
            for j in range(i + 1):
                w = gamma ** (t - j) * float(q[t] @ k[i]) * float(q[i] @ k[j])
                num += w * v[j]
                den += w
        o[t] = num / den if ratio else num
    return o


def decay_mask(n: int, gamma: float = 1.0):
    """D_g[t, i] = g^(t-i) for i <= t, else 0."""
    t = np.arange(n)
    diff = t[:, None] - t[None, :]
    return np.where(diff >= 0, float(gamma) ** np.maximum(diff, 0), 0.0)


def hla2_matrix(q, k, v, gamma: float = 1.0, ratio: bool = False):
    """Matrix form for one head (materialises n x n)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    A = q @ k.T
    Dg = decay_mask(n, gamma)
    L = np.tril(A)
    M = Dg * ((Dg * A) @ L.T)
    num = M @ v
    if ratio:
        return num / M.sum(axis=1, keepdims=True)
    return num


def ahla_matrix(q, k, v, ratio: bool = False, gamma: float = 1.0):
    """Matrix form for one head (materialises n x n)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    F = decay_mask(q.shape[0], gamma) * (q @ k.T)     # D_g * L (the mask zeroes i > t)
    M = F @ F
    num = M @ v
    if ratio:
        return num / M.sum(axis=1, keepdims=True)
    return num


def hla2_batched(q, k, v, H: int, gamma=None, ratio: bool = False):
    """Matrix form over [BH, n, d] inputs; gamma is None or a length-H array."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    out = np.empty(v.shape)
    for bh in range(q.shape[0]):
        g = 1.0 if gamma is None else float(gamma[bh % H])
        out[bh] = hla2_matrix(q[bh], k[bh], v[bh], g, ratio)
    return out


def ahla_batched(q, k, v, ratio: bool = False, H: int = 1, gamma=None):
    """Matrix form over [BH, n, d] inputs; gamma is None or a length-H array."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    out = np.empty(v.shape)
    for bh in range(q.shape[0]):
        g = 1.0 if gamma is None else float(gamma[bh % H])
        out[bh] = ahla_matrix(q[bh], k[bh], v[bh], ratio, g)
    return out
