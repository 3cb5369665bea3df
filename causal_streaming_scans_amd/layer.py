"""HLA as a differentiable operator and as an attention sub-layer.

The pages present HLA as a drop-in replacement for the attention sub-layer
of a Transformer block that needs only a kernel change ("Significancia" of
"Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
gist.science/es/paper/2510.27258).  This module wires the library's kernels
into PyTorch autograd:

* ``hla(q, k, v, variant, gamma)`` -- forward through ``hla_forward``,
  gradients through ``hla_backward``; both run in the library's HIP kernels;
* ``HLAAttention`` -- a sub-layer: bias-free q, k, v projections of the model
  dimension into heads, the HLA operator per head, heads merged, an output
  projection.  The four projections are plain GEMMs (torch, i.e. the ROCm
  BLAS libraries); every step of the operator itself runs in the library.

Variants with a backward: "hla2" (optional per-head decay), "hla2_ratio",
"ahla".  Inputs are bf16 or fp32 GPU tensors; d == dv.
"""
from __future__ import annotations

import torch

from . import hla_backward, hla_forward

_BACKWARD_VARIANTS = ("hla2", "hla2_ratio", "ahla")


class HLAFunction(torch.autograd.Function):
    """o = HLA(q, k, v); q, k, v: [B, H, n, d] contiguous, one dtype."""

    @staticmethod
    def forward(ctx, q, k, v, variant, gamma, chunk):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o = hla_forward(q, k, v, variant=variant, gamma=gamma, chunk=chunk)
        ctx.save_for_backward(q, k, v)
        ctx.variant, ctx.gamma = variant, gamma
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v = ctx.saved_tensors
        dq, dk, dv = hla_backward(q, k, v, do.contiguous(), variant=ctx.variant, gamma=ctx.gamma)
        return dq, dk, dv, None, None, None


def hla(q, k, v, variant: str = "hla2", gamma=None, chunk: int = 64):
    """Differentiable HLA over [B, H, n, d] tensors (see HLAFunction)."""
    if variant not in _BACKWARD_VARIANTS:
        raise ValueError(f"variant {variant!r} has no backward; one of {_BACKWARD_VARIANTS}")
    return HLAFunction.apply(q, k, v, variant, gamma, chunk)


class HLAAttention(torch.nn.Module):
    """Attention sub-layer with HLA in place of softmax attention.

    x: [B, n, d_model] -> [B, n, d_model].  Weights are bias-free linear maps
    (d_model -> heads * head_dim for q, k, v; heads * head_dim -> d_model for
    the output), initialised by torch's default; ``gamma`` is None or one
    decay per head (variant "hla2" only)."""

    def __init__(self, d_model: int, heads: int, head_dim: int, variant: str = "hla2",
                 gamma=None, chunk: int = 64, device=None, dtype=None):
        super().__init__()
        if variant not in _BACKWARD_VARIANTS:
            raise ValueError(f"variant {variant!r} has no backward; one of {_BACKWARD_VARIANTS}")
        kw = dict(bias=False, device=device, dtype=dtype)
        self.heads, self.head_dim = heads, head_dim
        self.variant, self.gamma, self.chunk = variant, gamma, chunk
        self.wq = torch.nn.Linear(d_model, heads * head_dim, **kw)
        self.wk = torch.nn.Linear(d_model, heads * head_dim, **kw)
        self.wv = torch.nn.Linear(d_model, heads * head_dim, **kw)
        self.wo = torch.nn.Linear(heads * head_dim, d_model, **kw)

    def _split(self, t):
        B, n, _ = t.shape
        return t.view(B, n, self.heads, self.head_dim).transpose(1, 2).contiguous()

    def forward(self, x):
        B, n, _ = x.shape
        q, k, v = self._split(self.wq(x)), self._split(self.wk(x)), self._split(self.wv(x))
        o = hla(q, k, v, self.variant, self.gamma, self.chunk)
        return self.wo(o.transpose(1, 2).reshape(B, n, self.heads * self.head_dim))
