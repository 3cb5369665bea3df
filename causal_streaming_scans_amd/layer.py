"""HLA as a differentiable operator and as an attention sub-layer.

The pages present HLA as a drop-in replacement for the attention sub-layer
of a Transformer block that needs only a kernel change ("Significancia" of
"Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
gist.science/es/paper/2510.27258).  This module wires the library's kernels
into PyTorch autograd:

* ``hla(q, k, v, variant, gamma)`` -- forward through ``hla_forward``,
  gradients through ``hla_backward``; both run in the library's HIP kernels;
  for "hla2" and "ahla" the forward also keeps the rows of its first chained
  pass (``hla_forward_z``: z_t = S_t q_t, y_t = P_t^T q_t), which the
  backward then does not recompute;
* ``HLAAttention`` -- a sub-layer: bias-free q, k, v projections of the model
  dimension into heads, the HLA operator per head, heads merged, an output
  projection.  The four projections are plain GEMMs (torch, i.e. the ROCm
  BLAS libraries); every step of the operator itself runs in the library.

Every variant has a backward ("hla2", "hla2_ratio", "ahla", "ahla_ratio",
"hla3", "hla3_ratio"), each with an optional per-head decay.  Inputs are
bf16 or fp32 GPU tensors; d == dv.  A decay given as a tensor that requires
grad receives dL/dgamma (HLA-2 forms only; the library's decay gradient,
summed over the batch); the library accepts decays in (0, 1] only, so a
learned decay must be kept in that range by its owner.
"""
from __future__ import annotations

import torch

from . import hla_backward, hla_forward, hla_forward_z

_BACKWARD_VARIANTS = ("hla2", "hla2_ratio", "ahla", "ahla_ratio", "hla3", "hla3_ratio")


class HLAFunction(torch.autograd.Function):
    """o = HLA(q, k, v); q, k, v: [B, H, n, d] contiguous, one dtype."""

    @staticmethod
    def forward(ctx, q, k, v, variant, gamma, chunk):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        ctx.gamma_is_tensor = isinstance(gamma, torch.Tensor)
        want_dg = ctx.gamma_is_tensor and ctx.needs_input_grad[4]
        # HLA-2 keeps the forward's keyed queries Z, AHLA its first pass Y, for
        # the backward, which then skips recomputing them (the decay
        # gradient's fp32 passes do not use them)
        z = None
        if variant in ("hla2", "ahla") and not want_dg:
            o, z = hla_forward_z(q, k, v, variant=variant, gamma=gamma, chunk=chunk)
        else:
            o = hla_forward(q, k, v, variant=variant, gamma=gamma, chunk=chunk)
        if ctx.gamma_is_tensor:
            ctx.save_for_backward(q, k, v, z, gamma)
        else:
            ctx.save_for_backward(q, k, v, z)
            ctx.gamma = gamma
        ctx.variant = variant
        return o

    @staticmethod
    def backward(ctx, do):
        if ctx.gamma_is_tensor:
            q, k, v, z, gamma = ctx.saved_tensors
        else:
            (q, k, v, z), gamma = ctx.saved_tensors, ctx.gamma
        want_dg = ctx.gamma_is_tensor and ctx.needs_input_grad[4]
        res = hla_backward(q, k, v, do.contiguous(), variant=ctx.variant, gamma=gamma,
                           dgamma=True if want_dg else None, z=None if want_dg else z)
        dgamma = None
        if want_dg:
            dgamma = res[3].to(gamma.device, gamma.dtype).reshape(gamma.shape)
        return res[0], res[1], res[2], None, dgamma, None


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
    decay per head (variant "hla2" only).  With ``learn_gamma`` the decays
    are an fp32 parameter trained through the library's decay gradient
    (its owner keeps them in (0, 1])."""

    def __init__(self, d_model: int, heads: int, head_dim: int, variant: str = "hla2",
                 gamma=None, chunk: int = 64, device=None, dtype=None, learn_gamma: bool = False):
        super().__init__()
        if variant not in _BACKWARD_VARIANTS:
            raise ValueError(f"variant {variant!r} has no backward; one of {_BACKWARD_VARIANTS}")
        kw = dict(bias=False, device=device, dtype=dtype)
        self.heads, self.head_dim = heads, head_dim
        self.variant, self.chunk = variant, chunk
        if learn_gamma:
            if gamma is None:
                raise ValueError("learn_gamma needs initial decays")
            gamma = torch.nn.Parameter(torch.as_tensor(gamma, dtype=torch.float32).reshape(heads).clone())
        self.gamma = gamma
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
