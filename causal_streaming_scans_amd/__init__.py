"""MI355X (gfx950) forward path of second-order Higher-order Linear Attention.

Thin Python binding over the C ABI of ``libhla.so`` (``include/hla.h``): it
only checks tensor shapes, allocates outputs and the workspace with PyTorch,
and passes raw device pointers plus the current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no CPU path, and
every entry point raises ``HLAError`` when the library is not built.

Operators (page: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)",
gist.science/es/paper/2510.27258, sections "1. HLA de Segundo Orden",
"2. ... (AHLA)", "4. ... Escaneos Asociativos"):

    hla2        o = tril(tril(QK^T) tril(QK^T)^T) V        (optional decay g_h)
    hla2_ratio  the same over its v == 1 denominator
    ahla        o = tril(QK^T) tril(QK^T) V
    ahla_ratio  the same over its v == 1 denominator
    hla3        o = tril(L L^T) L V, L = tril(QK^T)  (third order, section "3.
                HLA de Tercer Orden"; no decay, no ratio form)
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["HLAError", "VARIANTS", "NOALLOC_SCRATCH_BYTES", "load", "library_path", "ForwardPlan", "StepPlan",
           "BackwardPlan", "hla_forward", "hla_forward_stage", "hla_backward",
           "hla_step", "hla_unmasked_forward", "hla_forward_noalloc", "backward_workspace_bytes",
           "backward_default_seg_chunks", "unmasked_workspace_bytes",
           "state_floats", "workspace_bytes", "default_seg_chunks", "status_str"]

# bytes of the library's fixed workspace array behind hla_forward_noalloc
# (HLA_NOALLOC_SCRATCH_BYTES in include/hla.h)
NOALLOC_SCRATCH_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhla.so")
_lib = None

VARIANTS = {"hla2": 0, "hla2_ratio": 1, "ahla": 2, "ahla_ratio": 3, "hla3": 4, "hla3_ratio": 5}
_DTYPES = {"f32": 0, "bf16": 1}
MAX_DECAY_HEADS = 256


class HLAError(RuntimeError):
    """Raised for a missing library or a non-zero hla_status."""


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libhla.so (after torch, so that both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise HLAError(f"{_LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; "
                       f"g.build()'` or `python causal_streaming_scans_amd/build.py`")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    FP = ctypes.POINTER(ctypes.c_float)
    lib.hla_state_floats.argtypes = [I, I, I]
    lib.hla_state_floats.restype = Z
    lib.hla_default_seg_chunks.argtypes = [I, I, I, I, I, I]
    lib.hla_default_seg_chunks.restype = I
    lib.hla_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.hla_workspace_bytes.restype = Z
    lib.hla_forward.argtypes = [P, P, P, P, I, I, I, I, I, I, I, FP, I, I, P, P, P, Z, P]
    lib.hla_forward.restype = I
    lib.hla_forward_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, I, I, FP, I, I, P, P, P]
    lib.hla_forward_noalloc.restype = I
    lib.hla_forward_z.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, FP, I, I, P, P, P, Z, P]
    lib.hla_forward_z.restype = I
    lib.hla_forward_stage.argtypes = [I] + lib.hla_forward.argtypes
    lib.hla_forward_stage.restype = I
    lib.hla_step.argtypes = [P, P, P, P, I, I, I, I, I, I, FP, P, P]
    lib.hla_step.restype = I
    lib.hla_backward_default_seg_chunks.argtypes = [I, I, I]
    lib.hla_backward_default_seg_chunks.restype = I
    lib.hla_backward_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I]
    lib.hla_backward_workspace_bytes.restype = Z
    lib.hla_backward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, FP, P, I, P, Z, P]
    lib.hla_backward.restype = I
    lib.hla_backward_z.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, FP, I, P, Z, P]
    lib.hla_backward_z.restype = I
    lib.hla_unmasked_workspace_bytes.argtypes = [I, I, I, I]
    lib.hla_unmasked_workspace_bytes.restype = Z
    lib.hla_unmasked_forward.argtypes = [P, P, P, P, I, I, I, I, I, I, P, Z, P]
    lib.hla_unmasked_forward.restype = I
    lib.hla_status_str.argtypes = [I]
    lib.hla_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load().hla_status_str(int(code)).decode()


def _variant(v) -> int:
    if isinstance(v, str):
        if v not in VARIANTS:
            raise ValueError(f"unknown variant {v!r}; one of {sorted(VARIANTS)}")
        return VARIANTS[v]
    return int(v)


def state_floats(variant, d: int, dv: int) -> int:
    return int(load().hla_state_floats(_variant(variant), d, dv))


def default_seg_chunks(variant, B, H, n, d, chunk) -> int:
    return int(load().hla_default_seg_chunks(_variant(variant), B, H, n, d, chunk))


def workspace_bytes(variant, B, H, n, d, dv, chunk, seg_chunks=0) -> int:
    return int(load().hla_workspace_bytes(_variant(variant), B, H, n, d, dv, chunk, seg_chunks))


def backward_default_seg_chunks(B, H, n) -> int:
    return int(load().hla_backward_default_seg_chunks(B, H, n))


def backward_workspace_bytes(variant, B, H, n, d, dv, dtype="bf16", seg_chunks=0,
                             dgamma=False) -> int:
    return int(load().hla_backward_workspace_bytes(_variant(variant), B, H, n, d, dv,
                                                   _DTYPES[dtype], seg_chunks, int(bool(dgamma))))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return _DTYPES["bf16"]
    if t.dtype == torch.float32:
        return _DTYPES["f32"]
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _gamma_arg(gamma, H):
    if gamma is None:
        return None, None
    import numpy as np
    try:
        import torch
        if isinstance(gamma, torch.Tensor):
            gamma = gamma.detach().float().cpu().numpy()
    except ImportError:
        pass
    g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32).reshape(-1))
    if g.size != H:
        raise ValueError(f"gamma has {g.size} values, expected H = {H}")
    return g, g.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _check_device_tensor(name, t):
    if not t.is_cuda:
        raise HLAError(f"{name} must be a GPU tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise HLAError(f"{name} must be contiguous")


def _stream_ptr(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


class ForwardPlan:
    """The arguments of one forward pass, checked and marshalled once.

    ``run()`` enqueues the whole pass and ``stage(s)`` one stage of it (see
    hla_forward_stage), each as a single call into the library on the plan's
    stream; the plan keeps every tensor it points at alive.  For callers that
    launch the same shapes repeatedly (a timing loop, a decode server)."""

    def __init__(self, q, k, v, variant="hla2", gamma=None, chunk: int = 64, seg_chunks: int = 0,
                 state_in=None, state_out=None, out=None, workspace=None, stream=None,
                 staged=False, z=None):
        import torch
        lib = load()
        for name, t in (("q", q), ("k", k), ("v", v)):
            _check_device_tensor(name, t)
        if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
            raise HLAError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}: "
                           "expected [B,H,n,d], [B,H,n,d], [B,H,n,dv]")
        if not (q.dtype == k.dtype == v.dtype):
            raise HLAError("q, k, v must share one dtype")
        B, H, n, d = q.shape
        dv = v.shape[3]
        vid = _variant(variant)
        if out is None:
            out = torch.empty((B, H, n, dv), dtype=q.dtype, device=q.device)
        else:
            _check_device_tensor("out", out)
            if out.shape != (B, H, n, dv) or out.dtype != q.dtype:
                raise HLAError("out has the wrong shape or dtype")
        stf = state_floats(vid, d, dv)
        for name, t in (("state_in", state_in), ("state_out", state_out)):
            if t is not None:
                _check_device_tensor(name, t)
                if t.dtype != torch.float32 or t.numel() != B * H * stf:
                    raise HLAError(f"{name} must be fp32 with B*H*{stf} elements")
        need = workspace_bytes(vid, B, H, n, d, dv, chunk, seg_chunks)
        if workspace is None and need > 0:
            if staged:
                raise HLAError("hla_forward_stage needs the caller's workspace (shared by the stages)")
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        # the first chained pass's rows: Z (HLA-2, rows of d) or Y (AHLA, rows of dv)
        zlike = v if vid in (VARIANTS["ahla"], VARIANTS["ahla_ratio"]) else q
        if z is True:
            z = torch.empty_like(zlike)
        elif z is not None and z is not False:
            _check_device_tensor("z", z)
            if z.shape != zlike.shape or z.dtype != q.dtype:
                raise HLAError("z must have the shape and dtype of q (HLA-2) or v (AHLA)")
        else:
            z = None
        self.out = out
        self.z = z
        self._keep = (q, k, v, out, state_in, state_out, workspace, z)
        self._gamma, g_ptr = _gamma_arg(gamma, H)
        VP, CI = ctypes.c_void_p, ctypes.c_int
        ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
        self._args = (VP(q.data_ptr()), VP(k.data_ptr()), VP(v.data_ptr()), VP(out.data_ptr()),
                      CI(B), CI(H), CI(n), CI(d), CI(dv), CI(_dtype_code(q)), CI(vid), g_ptr,
                      CI(chunk), CI(seg_chunks),
                      VP(state_in.data_ptr() if state_in is not None else None),
                      VP(state_out.data_ptr() if state_out is not None else None),
                      VP(workspace.data_ptr() if workspace is not None else None),
                      ctypes.c_size_t(ws_len), _stream_ptr(stream, q.device))
        self._dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
        self._lib = lib

    def _call(self, fn, *lead):
        import torch
        if torch.cuda.current_device() == self._dev:
            rc = fn(*lead, *self._args)
        else:
            with torch.cuda.device(self._dev):
                rc = fn(*lead, *self._args)
        if rc != 0:
            raise HLAError(f"{fn.__name__} failed: {status_str(rc)} (code {rc})")
        return self.out

    def run(self):
        """o, or (o, z) when the plan was made with ``z`` (hla_forward_z)."""
        if self.z is None:
            return self._call(self._lib.hla_forward)
        self._call_z()
        return self.out, self.z

    def _call_z(self):
        import torch
        VP = ctypes.c_void_p
        args = self._args[:4] + (VP(self.z.data_ptr()),) + self._args[4:]
        if torch.cuda.current_device() == self._dev:
            rc = self._lib.hla_forward_z(*args)
        else:
            with torch.cuda.device(self._dev):
                rc = self._lib.hla_forward_z(*args)
        if rc != 0:
            raise HLAError(f"hla_forward_z failed: {status_str(rc)} (code {rc})")

    def stage(self, stage: int):
        return self._call(self._lib.hla_forward_stage, ctypes.c_int(int(stage)))


def _forward_call(stage, q, k, v, variant, gamma, chunk, seg_chunks, state_in, state_out, out,
                  workspace, stream):
    plan = ForwardPlan(q, k, v, variant, gamma, chunk, seg_chunks, state_in, state_out, out,
                       workspace, stream, staged=stage is not None)
    return plan.run() if stage is None else plan.stage(stage)


def hla_forward(q, k, v, variant="hla2", gamma=None, chunk: int = 64, seg_chunks: int = 0,
                state_in=None, state_out=None, out=None, workspace=None, stream=None):
    """Chunked HLA-2 / AHLA forward.  q, k: [B, H, n, d]; v: [B, H, n, dv];
    bf16 or fp32, contiguous, on one GPU.  gamma: None or H decays in (0, 1].
    state_in / state_out: None or fp32 [B, H, state_floats] device tensors.
    Returns o [B, H, n, dv] (``out`` if given)."""
    return _forward_call(None, q, k, v, variant, gamma, chunk, seg_chunks, state_in, state_out,
                         out, workspace, stream)


def hla_forward_z(q, k, v, variant="hla2", gamma=None, chunk: int = 64, seg_chunks: int = 0,
                  state_in=None, state_out=None, out=None, z=None, workspace=None, stream=None):
    """hla_forward that also returns the rows of its first chained pass, for
    hla_backward(..., z=z): HLA-2 forms the keyed queries z_t = S_t q_t
    ([B, H, n, d]), AHLA forms y_t = P_t^T q_t ([B, H, n, dv]); q's dtype,
    into ``z`` if given.  Returns (o, z)."""
    plan = ForwardPlan(q, k, v, variant, gamma, chunk, seg_chunks, state_in, state_out, out,
                       workspace, stream, z=True if z is None else z)
    return plan.run()


def hla_forward_stage(stage, q, k, v, variant="hla2", gamma=None, chunk: int = 64,
                      seg_chunks: int = 0, state_in=None, state_out=None, out=None,
                      workspace=None, stream=None):
    """One stage of hla_forward: 1 = segment summaries, 2 = up-sweep of the
    exclusive Blelloch scan over them, 3 = per-segment prefix from the
    up-sweep nodes and the chunked forward.  Stages 1, 2, 3 in order with the
    same arguments (and the same workspace and out) equal hla_forward."""
    return _forward_call(stage, q, k, v, variant, gamma, chunk, seg_chunks, state_in, state_out,
                         out, workspace, stream)


def hla_forward_noalloc(q, k, v, variant="hla2", gamma=None, chunk: int = 64,
                        seg_chunks: int = 0, state_in=None, state_out=None, out=None,
                        stream=None):
    """hla_forward with the library's fixed workspace array (no device
    allocation inside the call; see include/hla.h).  Same arguments as
    hla_forward, less ``workspace``.  Raises HLAError with
    HLA_ERR_WORKSPACE when the call needs more than that array holds."""
    import torch
    plan = ForwardPlan(q, k, v, variant, gamma, chunk, seg_chunks, state_in, state_out, out,
                       workspace=torch.empty(0, dtype=torch.uint8, device=q.device),
                       stream=stream)
    # the plan's arguments less the workspace pointer and size
    args = plan._args[:16] + plan._args[18:]
    with torch.cuda.device(plan._dev):
        rc = plan._lib.hla_forward_noalloc(*args)
    if rc != 0:
        raise HLAError(f"hla_forward_noalloc failed: {status_str(rc)} (code {rc})")
    return plan.out


class StepPlan:
    """One decode step's arguments, checked and marshalled once; ``run()``
    enqueues the step (state updated in place) as a single library call."""

    def __init__(self, q, k, v, state, variant="hla2", gamma=None, out=None, stream=None):
        import torch
        lib = load()
        for name, t in (("q", q), ("k", k), ("v", v), ("state", state)):
            _check_device_tensor(name, t)
        if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
            raise HLAError("expected q, k: [B, H, d], v: [B, H, dv]")
        B, H, d = q.shape
        dv = v.shape[2]
        vid = _variant(variant)
        if state.dtype != torch.float32 or state.numel() != B * H * state_floats(vid, d, dv):
            raise HLAError("state must be fp32 with B*H*state_floats elements")
        if out is None:
            out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
        self.out = out
        self._keep = (q, k, v, out, state)
        self._gamma, g_ptr = _gamma_arg(gamma, H)
        VP, CI = ctypes.c_void_p, ctypes.c_int
        self._args = (VP(q.data_ptr()), VP(k.data_ptr()), VP(v.data_ptr()), VP(out.data_ptr()),
                      CI(B), CI(H), CI(d), CI(dv), CI(_dtype_code(q)), CI(vid), g_ptr,
                      VP(state.data_ptr()), _stream_ptr(stream, q.device))
        self._dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
        self._lib = lib

    def run(self):
        import torch
        if torch.cuda.current_device() == self._dev:
            rc = self._lib.hla_step(*self._args)
        else:
            with torch.cuda.device(self._dev):
                rc = self._lib.hla_step(*self._args)
        if rc != 0:
            raise HLAError(f"hla_step failed: {status_str(rc)} (code {rc})")
        return self.out


def hla_step(q, k, v, state, variant="hla2", gamma=None, out=None, stream=None):
    """One decode step.  q, k: [B, H, d]; v: [B, H, dv]; state: fp32 device
    tensor with B*H*state_floats elements, updated in place.  Returns o."""
    return StepPlan(q, k, v, state, variant, gamma, out, stream).run()


class BackwardPlan:
    """The arguments of one backward pass (hla_backward), checked and
    marshalled once; ``run()`` enqueues it as a single library call and
    returns (dq, dk, dv), or (dq, dk, dv, dgamma) when ``dgamma`` is True or
    an fp32 [H] device tensor (HLA-2 forms: dL/dgamma_h summed over the
    batch, at the given decays, 1 when gamma is None)."""

    def __init__(self, q, k, v, do, variant="hla2", gamma=None, seg_chunks: int = 0,
                 dq=None, dk=None, dv=None, workspace=None, stream=None, dgamma=None, z=None):
        import torch
        lib = load()
        for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
            _check_device_tensor(name, t)
        if z is not None:
            _check_device_tensor("z", z)
            if z.shape != q.shape or z.dtype != q.dtype:
                raise HLAError("z must have the shape and dtype of q")
            if dgamma is not None and dgamma is not False:
                raise HLAError("dgamma is formed by hla_backward without z")
        if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or do.shape != q.shape:
            raise HLAError("expected q, k, v, do of one shape [B, H, n, d] (d == dv)")
        if not (q.dtype == k.dtype == v.dtype == do.dtype):
            raise HLAError("q, k, v, do must share one dtype")
        B, H, n, d = q.shape
        vid = _variant(variant)
        grads = []
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            if t is None:
                t = torch.empty_like(q)
            else:
                _check_device_tensor(name, t)
                if t.shape != q.shape or t.dtype != q.dtype:
                    raise HLAError(f"{name} has the wrong shape or dtype")
            grads.append(t)
        if dgamma is True:
            dgamma = torch.empty(H, dtype=torch.float32, device=q.device)
        elif dgamma is not None and dgamma is not False:
            _check_device_tensor("dgamma", dgamma)
            if dgamma.dtype != torch.float32 or dgamma.numel() != H:
                raise HLAError("dgamma must be an fp32 device tensor of H elements")
        else:
            dgamma = None
        self.dgamma = dgamma
        dtc = _dtype_code(q)
        need = int(lib.hla_backward_workspace_bytes(vid, B, H, n, d, d, dtc, seg_chunks,
                                                    int(dgamma is not None)))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        self.grads = tuple(grads)
        self._keep = (q, k, v, do, *grads, workspace, dgamma, z)
        self._gamma, g_ptr = _gamma_arg(gamma, H)
        VP, CI = ctypes.c_void_p, ctypes.c_int
        dg_ptr = VP(dgamma.data_ptr() if dgamma is not None else None)
        self._args = (VP(q.data_ptr()), VP(k.data_ptr()), VP(v.data_ptr()), VP(do.data_ptr()),
                      VP(grads[0].data_ptr()), VP(grads[1].data_ptr()), VP(grads[2].data_ptr()),
                      CI(B), CI(H), CI(n), CI(d), CI(d), CI(dtc), CI(vid), g_ptr, dg_ptr,
                      CI(seg_chunks),
                      VP(workspace.data_ptr()),
                      ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                      _stream_ptr(stream, q.device))
        self._dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
        self._lib = lib
        self._fn = lib.hla_backward
        if z is not None:
            # hla_backward_z: z after v, no dgamma
            self._args = self._args[:3] + (VP(z.data_ptr()),) + self._args[3:15] + self._args[16:]
            self._fn = lib.hla_backward_z

    def run(self):
        import torch
        if torch.cuda.current_device() == self._dev:
            rc = self._fn(*self._args)
        else:
            with torch.cuda.device(self._dev):
                rc = self._fn(*self._args)
        if rc != 0:
            raise HLAError(f"{self._fn.__name__} failed: {status_str(rc)} (code {rc})")
        return self.grads if self.dgamma is None else (*self.grads, self.dgamma)


def hla_backward(q, k, v, do, variant="hla2", gamma=None, seg_chunks: int = 0, dq=None, dk=None,
                 dv=None, workspace=None, stream=None, dgamma=None, z=None):
    """Gradients (dq, dk, dv) of the HLA-2 output with respect to q, k, v,
    given the upstream gradient do.  All four are [B, H, n, d] (d == dv), one
    dtype (bf16 or fp32), contiguous, on one GPU; gamma as in hla_forward.
    With ``dgamma`` (True or an fp32 [H] tensor) also returns dL/dgamma.
    With ``z`` (variant "hla2" or "ahla": the rows hla_forward_z returned
    for the same inputs and gamma) the backward skips recomputing them
    (hla_backward_z); not together with ``dgamma``."""
    return BackwardPlan(q, k, v, do, variant, gamma, seg_chunks, dq, dk, dv, workspace,
                        stream, dgamma, z).run()


def unmasked_workspace_bytes(B, H, n, d) -> int:
    return int(load().hla_unmasked_workspace_bytes(B, H, n, d))


def hla_unmasked_forward(q, k, v, variant="hla2", out=None, workspace=None, stream=None):
    """Unmasked (non-causal) operator over [B, H, n, d] tensors (d == dv, one
    dtype): "hla2" gives Q (K^T K)(Q^T V), "ahla" gives Q (K^T Q)(K^T V).
    Returns o [B, H, n, d] (``out`` if given)."""
    import torch
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise HLAError("expected q, k, v of one shape [B, H, n, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise HLAError("q, k, v must share one dtype")
    B, H, n, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_device_tensor("out", out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise HLAError("out has the wrong shape or dtype")
    need = int(lib.hla_unmasked_workspace_bytes(B, H, n, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    VP, CI = ctypes.c_void_p, ctypes.c_int
    with torch.cuda.device(q.device):
        rc = lib.hla_unmasked_forward(VP(q.data_ptr()), VP(k.data_ptr()), VP(v.data_ptr()),
                                      VP(out.data_ptr()), CI(B), CI(H), CI(n), CI(d),
                                      CI(_dtype_code(q)), CI(_variant(variant)),
                                      VP(workspace.data_ptr()),
                                      ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                      _stream_ptr(stream, q.device))
    if rc != 0:
        raise HLAError(f"hla_unmasked_forward failed: {status_str(rc)} (code {rc})")
    return out
