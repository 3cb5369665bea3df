"""The C ABI on a host without a GPU: the library loads, exports every
function include/hla.h declares, sizes are right, and argument validation
returns its error codes before any HIP call (nothing here launches work)."""
import ctypes
import os
import re

import numpy as np
import pytest

import causal_streaming_scans_amd as hla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hla.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_WS, ERR_DEV, ERR_ARG = range(7)
F32, BF16 = 0, 1
HLA2, HLA2_RATIO, AHLA, AHLA_RATIO = range(4)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hla.library_path()):
        import causal_streaming_scans_amd.build as b
        b.build()
    return hla.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hla_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"hla_forward", "hla_forward_stage", "hla_step", "hla_state_floats",
            "hla_workspace_bytes",
            "hla_default_seg_chunks", "hla_status_str"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(7):
        s = hla.status_str(code)
        assert s and s != "unknown status"
    assert hla.status_str(99) == "unknown status"


def test_state_floats(lib):
    assert hla.state_floats("hla2", 64, 64) == 64 * 64 + 64 * 64 + 64
    assert hla.state_floats("hla2_ratio", 16, 32) == 16 * 16 + 16 * 32 + 16
    assert hla.state_floats("ahla", 64, 64) == 2 * 64 * 64 + 2 * 64
    assert lib.hla_state_floats(7, 64, 64) == 0


def test_workspace_bytes(lib):
    # one segment: no workspace
    assert hla.workspace_bytes("hla2", 1, 1, 256, 16, 16, 32, 8) == 0
    # 4 segments -> 3 fp32 summaries per head, and room for as many up-sweep nodes
    sumf = 64 * 64 + 2 * 64 * 64 + 2 * 64
    assert hla.workspace_bytes("hla2", 2, 3, 1024, 64, 64, 64, 4) == 2 * 2 * 3 * 3 * sumf * 4
    # 3 segments (the last one partial) -> 2 summaries
    assert hla.workspace_bytes("ahla", 1, 1, 600, 64, 64, 64, 4) == 2 * 1 * 2 * sumf * 4


def test_default_segments_fill_the_chip(lib):
    # 128 heads x 4096 tokens: 4 segments of 16 chunks
    assert hla.default_seg_chunks("hla2_ratio", 8, 16, 4096, 64, 64) == 16
    # 32 heads x 65536 tokens: 16 segments of 64 chunks
    assert hla.default_seg_chunks("ahla", 1, 32, 65536, 64, 64) == 64
    # short sequences are never split below 8 chunks
    assert hla.default_seg_chunks("hla2", 1, 1, 256, 16, 32) == 8
    # d = 128: one workgroup per compute unit, 32 heads x 16384 tokens -> 8 segments
    assert hla.default_seg_chunks("hla2", 2, 16, 16384, 128, 64) == 32
    assert hla.default_seg_chunks("hla2", 2, 16, 16384, 64, 64) == 16


def _fwd(lib, q=1, k=1, v=1, o=1, B=1, H=1, n=64, d=64, dv=64, dtype=BF16, variant=HLA2,
         gamma=None, chunk=64, seg=0, si=None, so=None, ws=None, wsb=0):
    gp = None
    if gamma is not None:
        g = np.asarray(gamma, np.float32)
        gp = g.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    return lib.hla_forward(q, k, v, o, B, H, n, d, dv, dtype, variant, gp, chunk, seg, si, so,
                           ws, wsb, None)


def test_forward_validation_errors(lib):
    fake = 0x1000  # never dereferenced: every call below fails validation
    assert _fwd(lib, q=None, k=fake, v=fake, o=fake) == ERR_NULL
    assert _fwd(lib, q=fake, k=fake, v=fake, o=None) == ERR_NULL
    assert _fwd(lib, fake, fake, fake, fake, B=0) == ERR_SHAPE
    assert _fwd(lib, fake, fake, fake, fake, n=-1) == ERR_SHAPE
    assert _fwd(lib, fake, fake, fake, fake, d=0) == ERR_SHAPE
    assert _fwd(lib, fake, fake, fake, fake, dtype=5) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, variant=9) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, chunk=-16) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, seg=-1) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, chunk=48) == ERR_UNSUP
    assert _fwd(lib, fake, fake, fake, fake, d=48, dv=48) == ERR_UNSUP
    assert _fwd(lib, fake, fake, fake, fake, d=64, dv=32) == ERR_UNSUP
    assert _fwd(lib, fake, fake, fake, fake, d=128, dv=128, dtype=0) == ERR_UNSUP
    assert _fwd(lib, fake, fake, fake, fake, chunk=128) == ERR_UNSUP
    assert _fwd(lib, fake, fake, fake, fake, dtype=F32, d=128, dv=128, chunk=16) == ERR_UNSUP
    # decay: not for third order; gamma must lie in (0, 1]; H bounded
    assert _fwd(lib, fake, fake, fake, fake, variant=AHLA, gamma=[1.5]) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, gamma=[0.0]) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, gamma=[1.5]) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, gamma=[float("nan")]) == ERR_ARG
    assert _fwd(lib, fake, fake, fake, fake, H=300, gamma=[0.9] * 300) == ERR_UNSUP
    # workspace: needed when the sequence has several segments
    assert _fwd(lib, fake, fake, fake, fake, n=1024, seg=2, ws=None) == ERR_NULL
    need = hla.workspace_bytes("hla2", 1, 1, 1024, 64, 64, 64, 2)
    assert need > 0
    assert _fwd(lib, fake, fake, fake, fake, n=1024, seg=2, ws=fake, wsb=need - 1) == ERR_WS
    # the forward grid has one workgroup per (segment, head): at most 2^31 - 1
    assert _fwd(lib, fake, fake, fake, fake, B=64, H=1000, n=1 << 21, chunk=16, seg=1) == ERR_UNSUP
    # at dv = 128 the up-sweep has eight column slices per combine: nseg*B*H
    # up to 2^29 - 1 there (here 8389 * 64000 > 2^29), 2^30 - 1 otherwise
    big = dict(B=64, H=1000, n=8389 * 16, chunk=16, seg=1)
    assert _fwd(lib, fake, fake, fake, fake, d=128, dv=128, **big) == ERR_UNSUP
    assert _fwd(lib, fake, fake, fake, fake, **big) == ERR_NULL   # within the limit; no workspace
    # state_in may not alias state_out
    assert _fwd(lib, fake, fake, fake, fake, si=fake, so=fake) == ERR_ARG


def test_stage_validation_errors(lib):
    fake = 0x1000

    def stage(st, **kw):
        args = dict(B=1, H=1, n=64, d=64, dv=64, dtype=BF16, variant=HLA2, chunk=64, seg=0)
        args.update(kw)
        return lib.hla_forward_stage(st, fake, fake, fake, fake, args["B"], args["H"], args["n"],
                                     args["d"], args["dv"], args["dtype"], args["variant"], None,
                                     args["chunk"], args["seg"], None, None, None, 0, None)
    assert stage(0) == ERR_ARG
    assert stage(4) == ERR_ARG
    assert stage(1, B=0) == ERR_SHAPE
    assert stage(2, chunk=48) == ERR_UNSUP
    assert stage(3, n=1024, seg=2) == ERR_NULL   # workspace missing


def test_step_validation_errors(lib):
    fake = 0x1000

    def step(q=fake, st=fake, B=1, H=1, d=64, dv=64, dtype=BF16, variant=HLA2, gamma=None):
        gp = None
        if gamma is not None:
            g = np.asarray(gamma, np.float32)
            gp = g.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
        return lib.hla_step(q, fake, fake, fake, B, H, d, dv, dtype, variant, gp, st, None)

    assert step(q=None) == ERR_NULL
    assert step(st=None) == ERR_NULL
    assert step(B=0) == ERR_SHAPE
    assert step(d=24, dv=24) == ERR_UNSUP
    assert step(variant=AHLA_RATIO, gamma=[1.5]) == ERR_ARG
    assert step(gamma=[-0.5]) == ERR_ARG
    assert step(dtype=3) == ERR_ARG


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 16, 16)
    with pytest.raises(hla.HLAError):
        hla.hla_forward(x, x, x, chunk=16)


# ------------------------------------------------------------------ backward

def _bwd(lib, q=1, k=1, v=1, do=1, dq=1, dk=1, dv=1, B=1, H=2, n=128, d=64, dvd=64, dtype=BF16,
         variant=HLA2, gamma=None, dgamma=None, seg=0, ws=1, ws_bytes=1 << 40):
    P = ctypes.c_void_p
    g = None
    if gamma is not None:
        g = (ctypes.c_float * len(gamma))(*gamma)
    return lib.hla_backward(P(q), P(k), P(v), P(do), P(dq), P(dk), P(dv), B, H, n, d, dvd, dtype,
                            variant, g, P(dgamma), seg, P(ws), ws_bytes, None)


def test_backward_workspace_bytes(lib):
    # default segments: about 512 workgroups a pass, at least 2 chunks of 64 each
    assert lib.hla_backward_default_seg_chunks(4, 8, 2048) == 2
    assert lib.hla_backward_default_seg_chunks(8, 16, 4096) == 16
    assert lib.hla_backward_default_seg_chunks(1, 1, 256) == 2
    assert lib.hla_backward_default_seg_chunks(1, 1, 100) == 2 or \
        lib.hla_backward_default_seg_chunks(1, 1, 100) == 1
    B, H, n, d = 4, 8, 2048, 64
    g = lib.hla_backward_default_seg_chunks(B, H, n)
    nseg = -(-n // (64 * g))
    want = 2 * B * H * (nseg - 1) * d * d * 4 + 2 * B * H * n * d * 2
    dg = B * H * 64 * 8                    # fp64 partials of the decay gradient (HLA-2 forms)
    assert hla.backward_workspace_bytes("hla2", B, H, n, d, d, "bf16") == want + dg
    assert hla.backward_workspace_bytes("hla2", B, H, n, d, d, "f32", 32) == \
        2 * B * H * n * d * 4 + dg
    # the ratio form runs in fp32: 5 tensors, and with bf16 inputs 7 more
    # (fp32 copies of q, k, v, dO and fp32 gradients)
    want_ratio = want - 2 * B * H * n * d * 2 + 12 * B * H * n * d * 4
    assert hla.backward_workspace_bytes("hla2_ratio", B, H, n, d, d) == want_ratio + dg
    assert hla.backward_workspace_bytes("ahla_ratio", B, H, n, d, d) == \
        want_ratio + 2 * B * H * n * d * 4                   # Y1 and its gradient
    # third order keeps Y, Z, dZ, dY; its ratio form twelve fp32 tensors, plus
    # the seven widened copies and gradients for bf16 inputs
    assert hla.backward_workspace_bytes("hla3", B, H, n, d, d) == want + 2 * B * H * n * d * 2
    assert hla.backward_workspace_bytes("hla3_ratio", B, H, n, d, d) == \
        want - 2 * B * H * n * d * 2 + 19 * B * H * n * d * 4
    assert hla.backward_workspace_bytes("ahla", B, H, n, d, d) == want
    # with the decay gradient every pass runs in fp32: the two tensors in fp32
    # and, for bf16 inputs, the seven widened copies and gradients
    want_dg = want - 2 * B * H * n * d * 2 + 9 * B * H * n * d * 4
    assert hla.backward_workspace_bytes("hla2", B, H, n, d, d, "bf16", dgamma=True) == want_dg + dg
    assert hla.backward_workspace_bytes("hla2", B, H, n, d, d, "f32", 32, dgamma=True) == \
        2 * B * H * n * d * 4 + dg
    assert hla.backward_workspace_bytes("hla2_ratio", B, H, n, d, d, dgamma=True) == want_ratio + dg


def test_backward_validation(lib):
    assert _bwd(lib, n=0) == OK                      # nothing to do, nothing enqueued
    assert _bwd(lib, variant=HLA2_RATIO, ws_bytes=1) == ERR_WS
    assert _bwd(lib, variant=AHLA_RATIO, ws_bytes=1) == ERR_WS
    assert _bwd(lib, variant=4, dgamma=1) == ERR_UNSUP                    # no third-order decay gradient
    assert _bwd(lib, variant=6) == ERR_ARG
    assert _bwd(lib, variant=AHLA, dgamma=1) == ERR_UNSUP           # no AHLA decay gradient
    assert _bwd(lib, variant=AHLA_RATIO, dgamma=1) == ERR_UNSUP
    assert _bwd(lib, variant=AHLA, ws_bytes=1) == ERR_WS
    assert _bwd(lib, variant=9) == ERR_ARG
    assert _bwd(lib, dvd=32) == ERR_UNSUP
    assert _bwd(lib, d=48, dvd=48) == ERR_UNSUP
    assert _bwd(lib, d=256, dvd=256) == ERR_UNSUP
    assert _bwd(lib, dtype=5) == ERR_ARG
    assert _bwd(lib, B=0) == ERR_SHAPE
    assert _bwd(lib, n=-1) == ERR_SHAPE
    assert _bwd(lib, seg=-1) == ERR_ARG
    assert _bwd(lib, gamma=[0.9, 1.5]) == ERR_ARG
    assert _bwd(lib, gamma=[0.9, 0.0]) == ERR_ARG
    assert _bwd(lib, q=None) == ERR_NULL
    assert _bwd(lib, dv=None) == ERR_NULL
    assert _bwd(lib, ws=None) == ERR_NULL
    assert _bwd(lib, ws_bytes=1) == ERR_WS


# ---------------------------------------------------------------- third order

HLA3, HLA3_RATIO = 4, 5


def test_hla3_sizes_and_validation(lib):
    # P^KV per head, then the second-order state of (q, k, y); the ratio form
    # has that layout twice (the chain on v, then on unit values)
    one = 64 * 64 + (64 * 64 + 64 * 64 + 64)
    assert lib.hla_state_floats(HLA3, 64, 64) == one
    assert lib.hla_state_floats(HLA3_RATIO, 64, 64) == 2 * one
    B, H, n, d, chunk, seg = 2, 4, 1000, 64, 64, 4
    nseg = -(-n // (chunk * seg))
    scan = 2 * B * H * (nseg - 1) * (d * d + 2 * d * d + 2 * d) * 4
    g = lib.hla_backward_default_seg_chunks(B, H, n)
    nseg_la = -(-n // (64 * g))
    sums = B * H * (nseg_la - 1) * d * d * 4
    tensor = B * H * n * d * 4
    assert hla.workspace_bytes("hla3", B, H, n, d, d, chunk, seg) == scan + sums + 2 * tensor
    assert hla.workspace_bytes("hla3_ratio", B, H, n, d, d, chunk, seg) == scan + sums + 9 * tensor
    P = ctypes.c_void_p
    g2 = (ctypes.c_float * H)(*([0.9] * H))
    fwd = lambda **kw: lib.hla_forward(P(1), P(1), P(1), P(1), B, H, n, d, d, BF16,
                                       kw.get("variant", HLA3), kw.get("gamma"), chunk, seg,
                                       kw.get("si"), kw.get("so"), P(1), kw.get("ws", 1), None)
    assert fwd(ws=16) == ERR_WS
    assert fwd(gamma=g2, ws=16) == ERR_WS
    assert fwd(variant=HLA3_RATIO, ws=16) == ERR_WS
    bad = (ctypes.c_float * H)(*([1.5] * H))
    assert fwd(gamma=bad) == ERR_ARG
    assert lib.hla_step(P(1), P(1), P(1), P(1), B, H, d, d, BF16, HLA3, bad, P(1), None) == ERR_ARG


def test_binding_fails_loudly_without_the_library():
    """No CPU fallback: with libhla.so absent, every entry point raises."""
    import subprocess
    import sys
    code = ("import causal_streaming_scans_amd as h\n"
            "h._LIB_PATH = '/nonexistent/libhla.so'\n"
            "h._lib = None\n"
            "try:\n"
            "    h.load()\n"
            "except h.HLAError as e:\n"
            "    print('HLAError', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "HLAError" in r.stdout, r.stdout + r.stderr


def test_backward_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 64, 16)
    with pytest.raises(hla.HLAError):
        hla.hla_backward(x, x, x, x)


# ------------------------------------------------------------------ unmasked

def test_unmasked_sizes_and_validation(lib):
    P = ctypes.c_void_p
    B, H, n, d = 2, 4, 1000, 64
    nb = min(-(-512 // (B * H)), -(-n // 32), 64)
    assert lib.hla_unmasked_workspace_bytes(B, H, n, d) == \
        B * H * (2 * nb + 1) * d * d * 4 + B * H * d * d * 2
    assert hla.unmasked_workspace_bytes(1, 1, 10, 16) == (2 * 1 + 1) * 16 * 16 * 4 + 16 * 16 * 2
    assert lib.hla_unmasked_workspace_bytes(B, H, 0, d) == 0

    def fwd(q=1, k=1, v=1, o=1, B=B, H=H, n=n, d=d, dtype=BF16, variant=HLA2, ws=1,
            wsb=1 << 40):
        return lib.hla_unmasked_forward(P(q), P(k), P(v), P(o), B, H, n, d, dtype, variant,
                                        P(ws), wsb, None)
    assert fwd(n=0) == OK
    assert fwd(dtype=5) == ERR_ARG
    assert fwd(variant=9) == ERR_ARG
    assert fwd(variant=HLA2_RATIO) == ERR_UNSUP
    assert fwd(variant=AHLA_RATIO) == ERR_UNSUP
    assert fwd(variant=4) == ERR_UNSUP
    assert fwd(d=48) == ERR_UNSUP
    assert fwd(B=0) == ERR_SHAPE
    assert fwd(n=-1) == ERR_SHAPE
    assert fwd(q=None) == ERR_NULL
    assert fwd(ws=None) == ERR_NULL
    assert fwd(wsb=16) == ERR_WS


def test_noalloc_limit_and_validation(lib):
    """hla_forward_noalloc: the binding's size constant is the header's, a
    call needing more workspace than the fixed array holds is refused with
    HLA_ERR_WORKSPACE, and argument errors come first, as in hla_forward --
    all before any HIP call (the pointers here are never dereferenced)."""
    text = open(HEADER).read()
    m = re.search(r"#define HLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == hla.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    big = (64, 16, 8192, 128)
    assert hla.workspace_bytes("hla2", *big, 128, 16, 1) > hla.NOALLOC_SCRATCH_BYTES
    call = lambda B, H, n, d, dtype=BF16, variant=HLA2, chunk=16, seg=1: lib.hla_forward_noalloc(
        P(16), P(16), P(16), P(16), B, H, n, d, d, dtype, variant, None, chunk, seg, None, None,
        None)
    assert call(*big) == ERR_WS
    assert call(*big, dtype=7) == ERR_ARG
    assert call(64, 16, 8192, 0) == ERR_SHAPE
    assert call(1, 1, 100, 64, chunk=48) == ERR_UNSUP
    # no tokens: nothing to do, no workspace, no device work
    assert call(1, 1, 0, 64) == OK


# ------------------------------------------- keyed queries kept for the backward

def test_forward_z_validation(lib):
    """hla_forward_z: hla_forward's checks first, then its own (HLA-2 and
    AHLA forms, z needed for n > 0, z not one of q, k, v, o), all before any
    HIP call."""
    P = ctypes.c_void_p
    fake, z = 0x1000, 0x2000
    ws = hla.workspace_bytes("hla2", 1, 1, 4096, 64, 64, 64, 4)

    def fz(zp=z, q=fake, variant=HLA2, n=4096, wsb=ws, B=1):
        return lib.hla_forward_z(P(q), P(fake), P(fake), P(fake), P(zp), B, 1, n, 64, 64, BF16,
                                 variant, None, 64, 4, None, None, P(fake), wsb, None)
    assert fz(B=0) == ERR_SHAPE                 # the forward's own checks come first
    assert fz(wsb=1) == ERR_WS
    assert fz(variant=4, wsb=1 << 40) == ERR_UNSUP   # third order
    assert fz(zp=None) == ERR_NULL
    assert fz(zp=fake) == ERR_ARG               # z is q (and k, v, o)
    assert fz(zp=None, n=0) == OK               # no tokens, nothing enqueued


def test_backward_z_validation(lib):
    """hla_backward_z: HLA_HLA2 and HLA_AHLA, z needed for n > 0 and not an
    output."""
    P = ctypes.c_void_p

    def bz(z=5, variant=HLA2, n=128, dq=1, B=1):
        return lib.hla_backward_z(P(1), P(1), P(1), P(z), P(1), P(dq), P(2), P(3), B, 2, n, 64,
                                  64, BF16, variant, None, 0, P(1), 1 << 40, None)
    assert bz(B=0) == ERR_SHAPE
    assert bz(variant=HLA2_RATIO) == ERR_UNSUP
    assert bz(variant=AHLA_RATIO) == ERR_UNSUP
    assert bz(variant=9) == ERR_ARG
    assert bz(z=None) == ERR_NULL
    assert bz(z=1) == ERR_ARG                   # z is dq
    assert bz(z=None, n=0) == OK


def test_binding_forward_z_and_backward_z_checks():
    """The binding's own checks of z (no GPU call)."""
    import torch
    x = torch.zeros(1, 1, 8, 16)
    with pytest.raises(hla.HLAError):
        hla.hla_forward_z(x, x, x)                 # CPU tensors are refused first
    with pytest.raises(hla.HLAError):
        hla.hla_backward(x, x, x, x, z=x)
