"""Oracle for the HLA-2 / AHLA forward path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import, call, link or execute anything in this package.  The
product path (the HIP library and its Python binding) never touches it and
fails loudly when its own native library is missing.

Contents
--------
``hla_serial.c``   plain C fp64 serial recurrence in the page's summary form
                   (S^K, C^QV, m^Q, G, h for HLA-2; P^KV, E, m^K, n for AHLA);
                   OpenMP across heads.  Bound here through ctypes.
``definition.py``  brute-force masked-matrix definitions (n x n), fp64.
``chunk_scan.py``  the chunk-parallel algebra (segment summaries, semidirect
                   combine, exclusive Blelloch scan) written out in fp64 NumPy.
``backward.py``    gradients (dq, dk, dv) of the masked operators: the chain
                   rule applied to the n x n matrix form, fp64 NumPy.
``streaming_grad.py`` the same gradients as chains of causal linear
                   attention and their token-by-token recurrences, O(n d^2)
                   per head, for the long workloads; fp64 NumPy.
``third_order.py`` the masked third-order operator tril(L L^T) L V: loops,
                   matrix form and a serial recurrence, fp64 NumPy.
``unmasked.py``    the unmasked operators (A A^T) V and (A A) V: loops and
                   the matrix product, fp64 NumPy.

Source for every formula: "Resumen Tecnico: Atencion Lineal de Orden Superior
(HLA)", gist.science/es/paper/2510.27258, sections "1. HLA de Segundo Orden",
"2. ... (AHLA)" and "4. Entrenamiento Paralelo mediante Escaneos Asociativos".

Parity pins (tests/test_oracle_pins.py): brute force of the definition,
explicit double sums, the chained causal-linear-attention reduction, closed
forms for constant inputs, causality, homogeneity, ratio invariants and
scan == serial.  The decay law is a reading of the page (which only says
"with and without exponential decay"); it is pinned to its own brute-force
definition and to the closed-form geometric double sum, nothing more.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hla_serial.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, -O2, OpenMP).  No fast-math: the
    order of the fp64 sums is the one written in the source."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                     "-Wall", "-Wextra", "-o", tmp, _SRC], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P, L, I = ctypes.c_void_p, ctypes.c_long, ctypes.c_int
    lib.oracle_hla2.argtypes = [P, P, P, P, L, L, L, L, L, P, I, P, P, I]
    lib.oracle_hla2.restype = I
    lib.oracle_ahla.argtypes = [P, P, P, P, L, L, L, L, L, P, I, P, P, I]
    lib.oracle_ahla.restype = I
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    _lib = lib
    return lib


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def hla2_state_size(d: int, dv: int) -> int:
    return d * d + d * dv + d


def ahla_state_size(d: int, dv: int) -> int:
    return 2 * d * dv + 2 * d


def hla2(q, k, v, H=None, gamma=None, ratio=False, state_in=None,
         want_state=False, threads=0):
    """Serial fp64 HLA-2 over q, k: [BH, n, d], v: [BH, n, dv].

    Inputs are taken as exact fp32 values (pass bf16-rounded values upcast to
    fp32 to check a bf16 path).  gamma: None or length-H decay per head index
    h = bh % H.  state_in / state_out: [BH, d*d + d*dv + d] compact (S, W, u).
    Returns o (fp64) or (o, state_out)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    BH, n, d = q.shape
    dv = v.shape[2]
    H = H or BH
    o = np.empty((BH, n, dv), dtype=np.float64)
    g = None if gamma is None else np.ascontiguousarray(np.asarray(gamma, np.float64))
    si = None if state_in is None else np.ascontiguousarray(np.asarray(state_in, np.float64))
    so = np.empty((BH, hla2_state_size(d, dv))) if want_state else None
    rc = _load().oracle_hla2(_ptr(q), _ptr(k), _ptr(v), _ptr(o), BH, H, n, d, dv,
                             _ptr(g), int(bool(ratio)), _ptr(si), _ptr(so), int(threads))
    if rc:
        raise RuntimeError(f"oracle_hla2 failed ({rc})")
    return (o, so) if want_state else o


def ahla(q, k, v, ratio=False, state_in=None, want_state=False, threads=0, H=None,
         gamma=None):
    """Serial fp64 AHLA; state layout [BH, 2*d*dv + 2*d] = (P, E, m^K, n).
    gamma: None or length-H decay per head index h = bh % H (every summary
    decays by gamma per token)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    BH, n, d = q.shape
    dv = v.shape[2]
    H = H or BH
    o = np.empty((BH, n, dv), dtype=np.float64)
    g = None if gamma is None else np.ascontiguousarray(np.asarray(gamma, np.float64))
    si = None if state_in is None else np.ascontiguousarray(np.asarray(state_in, np.float64))
    so = np.empty((BH, ahla_state_size(d, dv))) if want_state else None
    rc = _load().oracle_ahla(_ptr(q), _ptr(k), _ptr(v), _ptr(o), BH, H, n, d, dv, _ptr(g),
                             int(bool(ratio)), _ptr(si), _ptr(so), int(threads))
    if rc:
        raise RuntimeError(f"oracle_ahla failed ({rc})")
    return (o, so) if want_state else o


def split_hla2_state(st, d, dv):
    """[..., d*d + d*dv + d] -> (S, W, u)."""
    st = np.asarray(st)
    S = st[..., :d * d].reshape(st.shape[:-1] + (d, d))
    W = st[..., d * d:d * d + d * dv].reshape(st.shape[:-1] + (d, dv))
    u = st[..., d * d + d * dv:]
    return S, W, u


def split_ahla_state(st, d, dv):
    st = np.asarray(st)
    P = st[..., :d * dv].reshape(st.shape[:-1] + (d, dv))
    E = st[..., d * dv:2 * d * dv].reshape(st.shape[:-1] + (d, dv))
    mK = st[..., 2 * d * dv:2 * d * dv + d]
    nk = st[..., 2 * d * dv + d:]
    return P, E, mK, nk
