"""Gradients of the masked HLA-2 / AHLA operators, fp64 -- TEST INFRASTRUCTURE ONLY.

Only the test suite and ``__graft_entry__.smoke()`` may use this module (see
``oracle/__init__.py``).  It shares no code with the HIP library.

The pages train HLA with the chunk-parallel scan ("4. Entrenamiento Paralelo
mediante Escaneos Asociativos" of "Resumen Tecnico: Atencion Lineal de Orden
Superior (HLA)", gist.science/es/paper/2510.27258), so the gradient that
training needs is the vector-Jacobian product of the forward operator.  The
pages print no backward formulas: what is written out here is the plain
definition, the chain rule applied to the masked matrix form of the operator
(materialising n x n matrices, so for small and medium n only).

Notation (one head): A = Q K^T, L = tril(A) (diagonal kept), D_g[t, i] =
g^(t-i) for i <= t else 0, given the upstream gradient dO of the output.

HLA-2 ("1. HLA de Segundo Orden"; decay reading: every prefix summary decays
by g per token):
    F = D_g * A,   N = F L^T,   M = D_g * N,   num = M V
    plain:  o = num
    ratio:  o = num / den,  den = M 1      (row sums)
AHLA ("2. ... (AHLA)"; with a decay every summary decays by g per token,
F = D_g * L):
    M = F F,  num = M V,  den = M 1

Gradient of the decay g (HLA-2): D_g enters twice, through F and through M.
With D'[t, i] = (t - i) g^(t-i-1) for i <= t (else 0), the derivative of
D_g, and dF, dM the gradients of F and M below,
    dL/dg = sum(dF * A * D') + sum(dM * N * D') .

Backward, in the order the chain rule visits the factors:
    ratio:  dnum = dO / den,  dden = -rowsum(dO * o) / den ;  else dnum = dO
    dV = M^T dnum
    dM = dnum V^T (+ dden 1^T)
    HLA-2:  dN = D_g * dM;  dF = dN L;  dL = dN^T F;  dA = D_g * dF + tril(dL)
    AHLA :  dM restricted to the lower triangle (M is lower-triangular);
            dF = dM F^T + F^T dM;  dA = D_g * dF
    dQ = dA K,  dK = dA^T Q
"""
from __future__ import annotations

import numpy as np

from .definition import decay_mask


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def hla2_vjp(q, k, v, do, gamma: float = 1.0, ratio: bool = False):
    """(dq, dk, dv) of HLA-2 for one head; q, k: [n, d], v, do: [n, dv]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    A = q @ k.T
    Dg = decay_mask(n, gamma)
    L = np.tril(A)
    F = Dg * A
    N = F @ L.T
    M = Dg * N
    num = M @ v
    if ratio:
        den = M.sum(axis=1, keepdims=True)
        o = num / den
        dnum = do / den
        dden = -(do * o).sum(axis=1, keepdims=True) / den
        dM = dnum @ v.T + dden            # dden broadcast over the columns (times 1^T)
    else:
        dnum = do
        dM = do @ v.T
    dv = M.T @ dnum
    dN = Dg * dM
    dF = dN @ L
    dL = dN.T @ F
    dA = Dg * dF + np.tril(dL)
    return dA @ k, dA.T @ q, dv


def hla2_dgamma(q, k, v, do, gamma: float = 1.0, ratio: bool = False) -> float:
    """dL/dg of HLA-2 for one head (L = sum(dO * o)), by the chain rule through
    the two decay masks of the matrix form."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    A = q @ k.T
    Dg = decay_mask(n, gamma)
    lag = np.arange(n)[:, None] - np.arange(n)[None, :]
    dD = np.where(lag >= 1, lag * float(gamma) ** np.maximum(lag - 1, 0), 0.0)
    L = np.tril(A)
    F = Dg * A
    N = F @ L.T
    M = Dg * N
    if ratio:
        den = M.sum(axis=1, keepdims=True)
        o = (M @ v) / den
        dM = (do / den) @ v.T - (do * o).sum(axis=1, keepdims=True) / den
    else:
        dM = do @ v.T
    dF = (Dg * dM) @ L
    return float((dF * A * dD).sum() + (dM * N * dD).sum())


def hla2_dgamma_batched(q, k, v, do, H: int, gamma=None, ratio: bool = False):
    """dL/dg_h over [BH, n, *] arrays: the per-(b, h) derivatives summed over
    the batch (bh = b * H + h).  Returns fp64 [H]."""
    out = np.zeros(H)
    for bh in range(q.shape[0]):
        g = 1.0 if gamma is None else float(gamma[bh % H])
        out[bh % H] += hla2_dgamma(q[bh], k[bh], v[bh], do[bh], g, ratio)
    return out


def ahla_vjp(q, k, v, do, ratio: bool = False, gamma: float = 1.0):
    """(dq, dk, dv) of AHLA for one head; with a decay, L below is the decayed
    lower-triangular factor F = D_g * tril(A) and M = F F."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Dg = decay_mask(q.shape[0], gamma)
    L = Dg * (q @ k.T)
    M = L @ L
    num = M @ v
    if ratio:
        den = M.sum(axis=1, keepdims=True)
        o = num / den
        dnum = do / den
        dden = -(do * o).sum(axis=1, keepdims=True) / den
        dM = np.tril(dnum @ v.T + dden)
    else:
        dnum = do
        dM = np.tril(do @ v.T)
    dv = M.T @ dnum
    dL = dM @ L.T + L.T @ dM
    dA = Dg * dL
    return dA @ k, dA.T @ q, dv


def hla2_vjp_batched(q, k, v, do, H: int, gamma=None, ratio: bool = False, heads=None):
    """Over [BH, n, *] arrays (or the listed head indices bh); gamma is None or
    a length-H array indexed by h = bh % H.  Returns fp64 (dq, dk, dv)."""
    bhs = range(q.shape[0]) if heads is None else heads
    res = [hla2_vjp(q[bh], k[bh], v[bh], do[bh],
                    1.0 if gamma is None else float(gamma[bh % H]), ratio) for bh in bhs]
    return tuple(np.stack([r[i] for r in res]) for i in range(3))


def ahla_vjp_batched(q, k, v, do, ratio: bool = False, heads=None, H: int = 1, gamma=None):
    bhs = range(q.shape[0]) if heads is None else heads
    res = [ahla_vjp(q[bh], k[bh], v[bh], do[bh], ratio,
                    1.0 if gamma is None else float(gamma[bh % H])) for bh in bhs]
    return tuple(np.stack([r[i] for r in res]) for i in range(3))
