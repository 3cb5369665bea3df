"""Chunk-parallel HLA-2 / AHLA forward by an exclusive Blelloch scan, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
(gist.science/es/paper/2510.27258), section "4. Entrenamiento Paralelo mediante
Escaneos Asociativos": token segments are concatenated by an associative
(semidirect-product) operator whose cross terms couple one segment's key moment
with the other's query-value moment; an exclusive Blelloch scan over segment
summaries then yields forward activations identical to the serial recurrence.
"Contribuciones Clave" item 2 adds the masked operators with exponential decay.

The page gives the structure but not the formulas.  This module writes out the
plainest reading (each step is checked against the serial oracle and the
brute-force definition by the test suite):

HLA-2 segment summary, from a zero state, over a segment of length l ending at
token e (g = decay, 1 for none):
    S = sum_i g^(e-i) k_i k_i^T                 C = sum_j g^(e-j) q_j v_j^T
    m = sum_j g^(e-j) q_j
    W = sum_j g^(2(e-j)) z_j v_j^T              u = sum_j g^(2(e-j)) z_j
    with z_j = sum_{i<=j in segment} g^(j-i) k_i (k_i . q_j)
Combine, segment A before segment B (the semidirect product):
    S = g^lB S_A + S_B ;  C = g^lB C_A + C_B ;  m = g^lB m_A + m_B
    W = g^(2 lB) W_A + W_B + g^lB S_A C_B
    u = g^(2 lB) u_A + u_B + g^lB S_A m_B ;      l = lA + lB
(W = S^K C^QV - G and u = S^K m^Q - h in the page's notation; the cross term
S_A C_B is the page's S^K_B C^QV_A written for W instead of G.)

AHLA segment summary from zero (every summary decays by g per token, as
for HLA-2; g = 1 is the undecayed operator): P = sum g^(e-j) k_j v_j^T,
mK = sum g^(e-j) k_j, E = sum_i g^(e-i) k_i y_i^T with
y_i = sum_{j<=i in segment} g^(i-j) (q_i . k_j) v_j,
nk = sum_i g^(e-i) k_i (q_i . mK_i), and the undecayed M = sum k q^T.
Combine, a = g^lB:
    P = a P_A + P_B ; mK = a mK_A + mK_B ; M = M_A + M_B
    E = a E_A + E_B + a M_B P_A ;  nk = a nk_A + nk_B + a M_B mK_A
(the cross term: a token i of B reads A's P decayed by g^(i - e_A), and its
row of E decays by g^(e - i) to the end, so the product is g^(e - e_A) = a
for every i: M_B is the plain sum).

Chunked forward inside a segment, carried state (S0, W0, u0), chunk tokens
tau = 0..c-1:
    Z = diag(g^(tau+1)) Q S0 + (D_g * Q K^T) K          (rows z_t = S_t q_t)
    P = D_{g^2} * tril(Q Z^T)
    O = diag(g^(2(tau+1))) Q W0 + P V ,  den = diag(g^(2(tau+1))) Q u0 + P 1
    S0 <- g^c S0 + K^T diag(g^(c-1-tau)) K
    W0 <- g^(2c) W0 + Z^T diag(g^(2(c-1-tau))) V ,  u0 likewise with 1
AHLA (F = D_g * tril(QK^T)): Y = diag(g^(tau+1)) Q P0 + F V ;
      O = diag(g^(tau+1)) Q E0 + F Y ; P0 <- g^c P0 + K^T diag(g^(c-1-tau)) V ;
      E0 <- g^c E0 + K^T diag(g^(c-1-tau)) Y (and the v == 1 column for mK, nk).
"""
from __future__ import annotations

import numpy as np


def _pw(g, e):
    return float(g) ** np.asarray(e, dtype=np.float64)


# --------------------------------------------------------------------- HLA-2

def hla2_zero(d, dv):
    return dict(S=np.zeros((d, d)), C=np.zeros((d, dv)), m=np.zeros(d),
                W=np.zeros((d, dv)), u=np.zeros(d), l=0)


def hla2_combine(A, B, g=1.0):
    """Semidirect combine; A is the earlier segment, B the later one."""
    gl, gl2 = _pw(g, B["l"]), _pw(g, 2 * B["l"])
    return dict(S=gl * A["S"] + B["S"],
                C=gl * A["C"] + B["C"],
                m=gl * A["m"] + B["m"],
                W=gl2 * A["W"] + B["W"] + gl * (A["S"] @ B["C"]),
                u=gl2 * A["u"] + B["u"] + gl * (A["S"] @ B["m"]),
                l=A["l"] + B["l"])


def _hla2_chunk(q, k, v, S0, W0, u0, g):
    """One chunk from carried state; returns (num, den, Z, S0', W0', u0')."""
    c = q.shape[0]
    tau = np.arange(c)
    Dg = np.where(tau[:, None] >= tau[None, :],
                  _pw(g, np.maximum(tau[:, None] - tau[None, :], 0)), 0.0)
    A = q @ k.T
    Z = _pw(g, tau + 1)[:, None] * (q @ S0) + (Dg * A) @ k
    P = (Dg * Dg) * np.tril(q @ Z.T)
    g2t = _pw(g, 2 * (tau + 1))[:, None]
    num = g2t * (q @ W0) + P @ v
    den = g2t[:, 0] * (q @ u0) + P.sum(axis=1)
    wk = _pw(g, c - 1 - tau)
    wz = _pw(g, 2 * (c - 1 - tau))
    S1 = _pw(g, c) * S0 + k.T @ (wk[:, None] * k)
    W1 = _pw(g, 2 * c) * W0 + Z.T @ (wz[:, None] * v)
    u1 = _pw(g, 2 * c) * u0 + Z.T @ wz
    return num, den, Z, S1, W1, u1


def hla2_segment_summary(q, k, v, chunk, g=1.0):
    """Summary of one segment from a zero state, built chunk by chunk."""
    n, d = q.shape
    dv = v.shape[1]
    S, W, u = np.zeros((d, d)), np.zeros((d, dv)), np.zeros(d)
    C, m = np.zeros((d, dv)), np.zeros(d)
    for c0 in range(0, n, chunk):
        qc, kc, vc = q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk]
        c = qc.shape[0]
        wq = _pw(g, c - 1 - np.arange(c))
        C = _pw(g, c) * C + qc.T @ (wq[:, None] * vc)
        m = _pw(g, c) * m + qc.T @ wq
        _, _, _, S, W, u = _hla2_chunk(qc, kc, vc, S, W, u, g)
    return dict(S=S, C=C, m=m, W=W, u=u, l=n)


def blelloch_exclusive(items, combine, zero):
    """Work-efficient exclusive scan (up-sweep then down-sweep) with a
    non-commutative operator; combine(A, B) has A earlier than B."""
    n = len(items)
    size = 1
    while size < n:
        size *= 2
    a = list(items) + [zero() for _ in range(size - n)]
    step = 1
    while step < size:                       # up-sweep
        for i in range(2 * step - 1, size, 2 * step):
            a[i] = combine(a[i - step], a[i])
        step *= 2
    a[size - 1] = zero()
    step = size // 2
    while step >= 1:                         # down-sweep
        for i in range(2 * step - 1, size, 2 * step):
            left = a[i - step]
            a[i - step] = a[i]
            a[i] = combine(a[i], left)
        step //= 2
    return a[:n]


def hla2_scan_forward(q, k, v, chunk, seg_chunks, gamma=1.0, ratio=False,
                      state_in=None):
    """One head. q, k: [n, d]; v: [n, dv].  Returns (o, state_out) where
    state_out = (S, W, u) at the end of the sequence."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, d = q.shape
    dv = v.shape[1]
    seg = chunk * seg_chunks
    bounds = [(s, min(s + seg, n)) for s in range(0, n, seg)] or [(0, 0)]
    sums = [hla2_segment_summary(q[a:b], k[a:b], v[a:b], chunk, gamma)
            for a, b in bounds]
    pref = blelloch_exclusive(sums, lambda A, B: hla2_combine(A, B, gamma),
                              lambda: hla2_zero(d, dv))
    if state_in is not None:
        S_in, W_in, u_in = state_in
        init = dict(S=S_in, C=np.zeros((d, dv)), m=np.zeros(d), W=W_in, u=u_in, l=0)
        pref = [hla2_combine(init, p, gamma) for p in pref]
    o = np.zeros((n, dv))
    S0 = W0 = u0 = None
    for (a, b), p in zip(bounds, pref):
        S0, W0, u0 = p["S"], p["W"], p["u"]
        for c0 in range(a, b, chunk):
            c1 = min(c0 + chunk, b)
            num, den, _, S0, W0, u0 = _hla2_chunk(q[c0:c1], k[c0:c1], v[c0:c1],
                                                  S0, W0, u0, gamma)
            o[c0:c1] = num / den[:, None] if ratio else num
    if S0 is None:
        S0, W0, u0 = np.zeros((d, d)), np.zeros((d, dv)), np.zeros(d)
    return o, (S0, W0, u0)


# ---------------------------------------------------------------------- AHLA

def ahla_zero(d, dv):
    return dict(P=np.zeros((d, dv)), E=np.zeros((d, dv)), M=np.zeros((d, d)),
                mK=np.zeros(d), nk=np.zeros(d), l=0)


def ahla_combine(A, B, g=1.0):
    """A earlier, B later; a = g^(tokens of B)."""
    a = 1.0 if g == 1.0 else float(g) ** B["l"]
    return dict(P=a * A["P"] + B["P"], M=A["M"] + B["M"], mK=a * A["mK"] + B["mK"],
                E=a * A["E"] + B["E"] + a * (B["M"] @ A["P"]),
                nk=a * A["nk"] + B["nk"] + a * (B["M"] @ A["mK"]),
                l=A.get("l", 0) + B.get("l", 0))


def _ahla_chunk(q, k, v, P0, E0, mK0, nk0, g=1.0):
    c = q.shape[0]
    tau = np.arange(c)
    F = np.tril(q @ k.T) * _pw(g, np.maximum(tau[:, None] - tau[None, :], 0))
    gt = _pw(g, tau + 1)
    Y = gt[:, None] * (q @ P0) + F @ v
    y1 = gt * (q @ mK0) + F.sum(axis=1)
    num = gt[:, None] * (q @ E0) + F @ Y
    den = gt * (q @ nk0) + F @ y1
    kw = _pw(g, c - 1 - tau)[:, None] * k
    gc = float(g) ** c
    return (num, den, gc * P0 + kw.T @ v, gc * E0 + kw.T @ Y, gc * mK0 + kw.sum(axis=0),
            gc * nk0 + kw.T @ y1)


def ahla_segment_summary(q, k, v, chunk, g=1.0):
    n, d = q.shape
    dv = v.shape[1]
    s = ahla_zero(d, dv)
    P, E, mK, nk = s["P"], s["E"], s["mK"], s["nk"]
    for c0 in range(0, n, chunk):
        qc, kc, vc = q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk]
        _, _, P, E, mK, nk = _ahla_chunk(qc, kc, vc, P, E, mK, nk, g)
    return dict(P=P, E=E, M=k.T @ q, mK=mK, nk=nk, l=n)


def ahla_scan_forward(q, k, v, chunk, seg_chunks, ratio=False, state_in=None, gamma=1.0):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, d = q.shape
    dv = v.shape[1]
    seg = chunk * seg_chunks
    bounds = [(s, min(s + seg, n)) for s in range(0, n, seg)] or [(0, 0)]
    sums = [ahla_segment_summary(q[a:b], k[a:b], v[a:b], chunk, gamma) for a, b in bounds]
    comb = lambda A, B: ahla_combine(A, B, gamma)
    pref = blelloch_exclusive(sums, comb, lambda: ahla_zero(d, dv))
    if state_in is not None:
        P_in, E_in, mK_in, nk_in = state_in
        init = dict(P=P_in, E=E_in, M=np.zeros((d, d)), mK=mK_in, nk=nk_in, l=0)
        pref = [comb(init, p) for p in pref]
    o = np.zeros((n, dv))
    st = None
    for (a, b), p in zip(bounds, pref):
        st = (p["P"], p["E"], p["mK"], p["nk"])
        for c0 in range(a, b, chunk):
            c1 = min(c0 + chunk, b)
            num, den, *st = _ahla_chunk(q[c0:c1], k[c0:c1], v[c0:c1], *st, g=gamma)
            o[c0:c1] = num / den[:, None] if ratio else num
    if st is None:
        st = (np.zeros((d, dv)), np.zeros((d, dv)), np.zeros(d), np.zeros(d))
    return o, tuple(st)
