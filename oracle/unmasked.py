"""Unmasked (non-causal) second-order operators, fp64 -- TEST INFRASTRUCTURE ONLY.

Only the test suite may use this module (see ``oracle/__init__.py``); it
shares no code with the HIP library.

Page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
(gist.science/es/paper/2510.27258).  Without its causal masks the operator of
"1. HLA de Segundo Orden" is the plain product of the attention matrix with
its transpose, and the operator of "2. ... (AHLA)" the product of the
attention matrix with itself:

    A = Q K^T,   HLA-2: o = (A A^T) V,   AHLA: o = (A A) V,

i.e. o_t = sum_j sum_s A[t,s] A[j,s] v_j and o_t = sum_s A[t,s] sum_j A[s,j] v_j
over all tokens.  Two forms: explicit loops (tiny n) and the matrix product,
evaluated right to left (A (A^T V), A (A V)) so that it stays O(n^2 d).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def hla2_unmasked_loops(q, k, v):
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]))
    for t in range(n):
        for j in range(n):
            for s in range(n):
                o[t] += float(q[t] @ k[s]) * float(q[j] @ k[s]) * v[j]
    return o


def ahla_unmasked_loops(q, k, v):
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]))
    for t in range(n):
        for s in range(n):
            for j in range(n):
                o[t] += float(q[t] @ k[s]) * float(q[s] @ k[j]) * v[j]
    return o


def hla2_unmasked(q, k, v):
    """(A A^T) V for one head, A = Q K^T."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    A = q @ k.T
    return A @ (A.T @ v)


def ahla_unmasked(q, k, v):
    """(A A) V for one head."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    A = q @ k.T
    return A @ (A @ v)


def unmasked_batched(q, k, v, variant: str = "hla2", heads=None):
    """Over [BH, n, d] arrays (or the listed head indices)."""
    f = hla2_unmasked if variant == "hla2" else ahla_unmasked
    bhs = range(q.shape[0]) if heads is None else heads
    return np.stack([f(q[bh], k[bh], v[bh]) for bh in bhs])
