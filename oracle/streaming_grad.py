"""Gradients of HLA-2 and AHLA in linear time, fp64 -- TEST INFRASTRUCTURE ONLY.

Only the test suite may use this module (see ``oracle/__init__.py``); it
shares no code with the HIP library.

The matrix-form gradients in ``backward.py`` materialise n x n matrices, so
they serve sequences of a few thousand tokens.  For the long workloads
(n = 16384 at d = 128, n = 65536) the same gradients are written here as
token-by-token recurrences, which cost O(n d^2) per head.

Both operators are chains of causal linear attention ("1. HLA de Segundo
Orden" and "2. ... (AHLA)" of "Resumen Tecnico: Atencion Lineal de Orden
Superior (HLA)", gist.science/es/paper/2510.27258; decay reading: every
prefix summary decays by g per token):

    LA_g(a, b, c)_t = sum_{s <= t} g^(t-s) (a_t . b_s) c_s
    HLA-2:  Z = LA_g(Q, K, K),   O = LA_{g^2}(Q, Z, V)
    AHLA :  Y = LA_g(Q, K, V),   O = LA_g(Q, K, Y)

(ratio forms: V widened by a ones column; the last column of the chain's
output is the denominator.)  Differentiating LA_g term by term gives three
sums of the same kind, two of them over later tokens:

    da_t = sum_{s <= t} g^(t-s) (dout_t . c_s) b_s   = LA_g(dout, c, b)_t
    db_s = sum_{t >= s} g^(t-s) (dout_t . c_s) a_t   = RLA_g(c, dout, a)_s
    dc_s = sum_{t >= s} g^(t-s) (a_t . b_s) dout_t   = RLA_g(b, a, dout)_s

with RLA_g(x, y, z)_s = sum_{t >= s} g^(t-s) (x_s . y_t) z_t.  Each sum is
evaluated by its own state recurrence (P <- g P + b_s c_s^T, out_t = P^T a_t;
the anti-causal one runs from the last token down).  Pinned element by
element to the matrix-form chain rule in tests/test_oracle_streaming_grad.py.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _gammas(BH: int, H: int, gamma) -> np.ndarray:
    if gamma is None:
        return np.ones(BH)
    return np.array([float(gamma[bh % H]) for bh in range(BH)])


def causal_la(a, b, c, g):
    """LA_g(a, b, c) over [BH, n, *] arrays with one decay per head (g: [BH]):
    the state P = sum_{s <= t} g^(t-s) b_s c_s^T, updated token by token."""
    BH, n, _ = a.shape
    P = np.zeros((BH, b.shape[2], c.shape[2]))
    out = np.empty((BH, n, c.shape[2]))
    gg = g[:, None, None]
    for t in range(n):
        P = gg * P + b[:, t, :, None] * c[:, t, None, :]
        out[:, t] = np.matmul(a[:, t, None, :], P)[:, 0]
    return out


def anti_causal_la(x, y, z, g):
    """RLA_g(x, y, z)_s = sum_{t >= s} g^(t-s) (x_s . y_t) z_t over [BH, n, *]
    arrays: the state R = sum_{t >= s} g^(t-s) y_t z_t^T, from the last token
    down."""
    BH, n, _ = x.shape
    R = np.zeros((BH, y.shape[2], z.shape[2]))
    out = np.empty((BH, n, z.shape[2]))
    gg = g[:, None, None]
    for s in range(n - 1, -1, -1):
        R = gg * R + y[:, s, :, None] * z[:, s, None, :]
        out[:, s] = np.matmul(x[:, s, None, :], R)[:, 0]
    return out


def la_vjp(a, b, c, dout, g):
    """(da, db, dc) of out = LA_g(a, b, c) given dout."""
    return (causal_la(dout, c, b, g), anti_causal_la(c, dout, a, g),
            anti_causal_la(b, a, dout, g))


def _widen(v):
    return np.concatenate([v, np.ones(v.shape[:2] + (1,))], axis=2)


def _ratio_upstream(num, do):
    """Upstream gradient of the widened numerator [num, den] for o = num / den."""
    den = num[:, :, -1:]
    o = num[:, :, :-1] / den
    dden = -(do * o).sum(axis=2, keepdims=True) / den
    return np.concatenate([do / den, dden], axis=2)


def hla2_vjp_streaming(q, k, v, do, H: int = 1, gamma=None, ratio: bool = False):
    """(dq, dk, dv) of HLA-2 over [BH, n, *] arrays in O(n d^2) per head."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    g = _gammas(q.shape[0], H, gamma)
    vw = _widen(v) if ratio else v
    z = causal_la(q, k, k, g)
    if ratio:
        dnum = _ratio_upstream(causal_la(q, z, vw, g * g), do)
    else:
        dnum = do
    dq2, dz, dvw = la_vjp(q, z, vw, dnum, g * g)
    dq1, dk_b, dk_c = la_vjp(q, k, k, dz, g)
    dv = dvw[:, :, :-1] if ratio else dvw
    return dq1 + dq2, dk_b + dk_c, dv


def ahla_vjp_streaming(q, k, v, do, H: int = 1, gamma=None, ratio: bool = False):
    """(dq, dk, dv) of AHLA over [BH, n, *] arrays in O(n d^2) per head."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    g = _gammas(q.shape[0], H, gamma)
    vw = _widen(v) if ratio else v
    y = causal_la(q, k, vw, g)
    if ratio:
        dnum = _ratio_upstream(causal_la(q, k, y, g), do)
    else:
        dnum = do
    dq2, dk2, dy = la_vjp(q, k, y, dnum, g)
    dq1, dk1, dvw = la_vjp(q, k, vw, dy, g)
    dv = dvw[:, :, :-1] if ratio else dvw
    return dq1 + dq2, dk1 + dk2, dv
