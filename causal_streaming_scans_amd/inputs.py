"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random numbers and
rounds them to the storage type.  It imports nothing from the rest of the
package, so the oracle side of a check can use it without touching the HIP
library.

Recipe (one generator per workload, NumPy PCG64 seeded with ``seed``; draws in
fp64 in the order q, k, v, then gamma, then any decode tokens; rounded to fp32,
then to bf16 with round-to-nearest-even where the workload is bf16):

  ``normal_scaled``  q, k, v ~ N(0, 1/d)                       (small fp32 case)
  ``l2norm``         q, k = L2-normalised rows of N(0, 1); v ~ N(0, 1)
  ``uniform_pos``    q, k ~ U[0, 1)/sqrt(d) (positive scores, so the masked
                     ratio denominator stays > 0); v ~ N(0, 1)
  gamma (per head)   U[0.95, 0.999]

The named workloads mirror the configurations the path is measured on.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def bf16_round(x) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding the exact
    bf16 value.  Inputs here are finite."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x_exact_bf16: np.ndarray) -> np.ndarray:
    """fp32 arrays holding bf16 values -> their uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x_exact_bf16, dtype=np.float32))
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Workload:
    name: str
    variant: str          # "hla2", "hla2_ratio", "ahla"
    B: int
    H: int
    n: int
    d: int
    dv: int
    dtype: str            # "f32" or "bf16"
    dist: str             # "normal_scaled", "l2norm", "uniform_pos"
    chunk: int
    decay: bool = False
    decode_tokens: int = 0
    seed: int = 0


WORKLOADS = {
    "small_f32": Workload("HLA-2 B=1 H=1 n=256 d=dv=16 fp32 chunk=32", "hla2",
                          1, 1, 256, 16, 16, "f32", "normal_scaled", 32, seed=1001),
    "hla2_n2048": Workload("HLA-2 B=4 H=8 n=2048 d=dv=64 bf16 chunk=64", "hla2",
                           4, 8, 2048, 64, 64, "bf16", "l2norm", 64, seed=1002),
    "ratio_n4096": Workload("HLA-2 ratio B=8 H=16 n=4096 d=dv=64 bf16", "hla2_ratio",
                            8, 16, 4096, 64, 64, "bf16", "uniform_pos", 64, seed=1003),
    "decay_n16384": Workload("HLA-2 decay B=2 H=16 n=16384 d=dv=128 bf16", "hla2",
                             2, 16, 16384, 128, 128, "bf16", "l2norm", 64, decay=True,
                             seed=1004),
    "ahla_n65536": Workload("AHLA B=1 H=32 n=65536 d=dv=64 bf16 + 1024 decode", "ahla",
                            1, 32, 65536, 64, 64, "bf16", "l2norm", 64,
                            decode_tokens=1024, seed=1005),
}


def _draw(rng, dist, BH, n, d, dv):
    if dist == "normal_scaled":
        s = 1.0 / np.sqrt(d)
        q = rng.standard_normal((BH, n, d)) * s
        k = rng.standard_normal((BH, n, d)) * s
        v = rng.standard_normal((BH, n, dv)) * (1.0 / np.sqrt(dv))
    elif dist == "l2norm":
        q = rng.standard_normal((BH, n, d))
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((BH, n, d))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((BH, n, dv))
    elif dist == "uniform_pos":
        s = 1.0 / np.sqrt(d)
        q = rng.random((BH, n, d)) * s
        k = rng.random((BH, n, d)) * s
        v = rng.standard_normal((BH, n, dv))
    else:
        raise ValueError(dist)
    return q, k, v


def _store(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def make_inputs(B, H, n, d, dv, dtype="bf16", dist="l2norm", seed=0,
                decay=False, decode_tokens=0):
    """Return a dict of fp32 arrays holding exactly the stored values:
    q, k [B*H, n, d], v [B*H, n, dv], gamma [H] or None, and for decode
    q_dec, k_dec [decode_tokens, B*H, d], v_dec [decode_tokens, B*H, dv]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    BH = B * H
    q, k, v = _draw(rng, dist, BH, n, d, dv)
    out = dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype))
    del q, k, v
    out["gamma"] = (rng.uniform(0.95, 0.999, H).astype(np.float32) if decay else None)
    if decode_tokens:
        qd, kd, vd = _draw(rng, dist, BH, decode_tokens, d, dv)
        out["q_dec"] = np.ascontiguousarray(_store(qd, dtype).transpose(1, 0, 2))
        out["k_dec"] = np.ascontiguousarray(_store(kd, dtype).transpose(1, 0, 2))
        out["v_dec"] = np.ascontiguousarray(_store(vd, dtype).transpose(1, 0, 2))
    return out


def make_upstream_grad(BH, n, dv, dtype="bf16", seed=0):
    """Upstream gradient dL/do for a backward pass: N(0, 1) entries,
    [B*H, n, dv], from its own PCG64 stream, rounded like the inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _store(rng.standard_normal((BH, n, dv)), dtype)


def workload_inputs(key: str, **overrides):
    w = WORKLOADS[key]
    kw = dict(B=w.B, H=w.H, n=w.n, d=w.d, dv=w.dv, dtype=w.dtype, dist=w.dist,
              seed=w.seed, decay=w.decay, decode_tokens=w.decode_tokens)
    kw.update(overrides)
    return make_inputs(**kw)
