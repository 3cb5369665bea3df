"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C ABI's host side (causal_streaming_scans_amd/csrc/hla_api.cpp: argument
  validation, workspace carving, pass lists, parameter blocks) built with g++
  and the sanitizers, linked against stand-ins for the kernel lookups whose
  launches only record their arguments (tests/sanitize/abi_driver.cpp): every
  variant, dtype, decay, several d and n (0, 1, ragged), forward, stages,
  decode and backward, with workspaces of exactly the advertised size.  Any
  sanitizer report, any device pointer outside the caller's buffers and
  workspace, or any unexpected status fails the test.
* The fp64 serial oracle (oracle/hla_serial.c) built the same way and run on
  seeded inputs (tests/sanitize/oracle_driver.c); its outputs and states must
  equal those of the ordinary build.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r


def test_c_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    r = _run(["g++", "-std=c++17", "-Wall", *SAN, "-D__HIP_PLATFORM_AMD__",
              "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
              "-I", os.path.join(ROOT, "causal_streaming_scans_amd", "csrc"),
              os.path.join(ROOT, "causal_streaming_scans_amd", "csrc", "hla_api.cpp"),
              os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe])
    assert r.returncode == 0, r.stderr[-3000:]
    r = _run([exe], env=ENV, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    assert "pointers outside 0, failed expectations 0" in out


def test_oracle_under_sanitizers_equals_plain_build(tmp_path):
    exe = str(tmp_path / "oracle_san")
    r = _run(["gcc", "-std=c11", "-Wall", *SAN, "-fopenmp",
              os.path.join(ROOT, "oracle", "hla_serial.c"),
              os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"])
    assert r.returncode == 0, r.stderr[-3000:]
    rng = np.random.default_rng(61)
    BH, H, n, d, dv = 4, 2, 37, 5, 3
    q = (rng.random((BH, n, d)) / np.sqrt(d)).astype(np.float32)
    k = (rng.random((BH, n, d)) / np.sqrt(d)).astype(np.float32)
    v = rng.standard_normal((BH, n, dv)).astype(np.float32)
    g = np.array([0.9, 0.97])
    s2 = d * d + d * dv + d
    sa = 2 * d * dv + 2 * d
    si2 = rng.random((BH, s2)) * 0.1
    sia = rng.random((BH, sa)) * 0.1
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(fin, "wb") as f:
        f.write(np.array([BH, H, n, d, dv], np.int64).tobytes())
        for a in (q, k, v, g, si2, sia):
            f.write(np.ascontiguousarray(a).tobytes())
    r = _run([exe, fin, fout], env=dict(ENV, OMP_NUM_THREADS="1"), timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    got = np.fromfile(fout, np.float64)
    want = []
    for fam in ("hla2", "ahla"):
        for ratio in (False, True):
            for decay in (False, True):
                gam = g if decay else None
                if fam == "hla2":
                    o, st = oracle.hla2(q, k, v, H=H, gamma=gam, ratio=ratio, state_in=si2,
                                        want_state=True)
                else:
                    o, st = oracle.ahla(q, k, v, ratio=ratio, state_in=sia, want_state=True, H=H,
                                        gamma=gam)
                want += [o.reshape(-1), st.reshape(-1)]
    want = np.concatenate(want)
    assert got.shape == want.shape
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)
