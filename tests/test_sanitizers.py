"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI shim (gated_deltanet_chunked_gdn_amd/csrc/gdn_abi.cpp) is built with
g++ against host stand-ins for the device launchers (tests/sanitize/stubs.cpp)
and driven by tests/sanitize/abi_driver.cpp: status strings, workspace sizes
over a grid of problems up to the documented limits, and every entry point
with invalid and with valid-looking arguments.  The fp64 oracle
(oracle/gdn_oracle.c) is built with gcc and driven by
tests/sanitize/oracle_driver.c (dense and packed inputs, 1 and 3 threads, which
must agree bit for bit); its last forward is compared with the regular
liboracle build.  Any sanitizer report aborts the driver (no recovery).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_deltanet_chunked_gdn_amd", "csrc")
FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_shim_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    r = _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
              "-I" + CSRC, *FLAGS, os.path.join(CSRC, "gdn_abi.cpp"), os.path.join(SAN, "stubs.cpp"),
              os.path.join(SAN, "abi_driver.cpp"), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
              "-o", exe])
    assert r.returncode == 0, r.stderr[-4000:]
    r = _run([exe], env=ENV)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert r.stdout.strip().splitlines()[-1].startswith("ok:")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    r = _run(["gcc", "-std=c11", *FLAGS, "-pthread", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
              os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    assert r.returncode == 0, r.stderr[-4000:]
    dump = str(tmp_path / "last.bin")
    r = _run([exe, dump], env=ENV)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert r.stdout.strip().splitlines()[-1].startswith("ok:")
    # the sanitized build computes what the regular build computes (last case:
    # sequences of 33 and 67 tokens, H = 2, d_k = 12, d_v = 10, scale 0.5)
    cu = np.array([0, 33, 100])
    T, H, Dk, Dv, N = 100, 2, 12, 10, 2
    x = np.fromfile(dump, dtype=np.float64)
    sizes = [T * H * Dk, T * H * Dk, T * H * Dv, T * H, T * H, N * H * Dk * Dv, T * H * Dv, N * H * Dk * Dv]
    parts = np.split(x, np.cumsum(sizes)[:-1])
    q, k, v = parts[0].reshape(T, H, Dk), parts[1].reshape(T, H, Dk), parts[2].reshape(T, H, Dv)
    g, beta, S0 = parts[3].reshape(T, H), parts[4].reshape(T, H), parts[5].reshape(N, H, Dk, Dv)
    o, Sf = oracle.fwd(q, k, v, g, beta, cu_seqlens=cu, S0=S0, scale=0.5)
    np.testing.assert_allclose(parts[6].reshape(T, H, Dv), o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(parts[7].reshape(N, H, Dk, Dv), Sf, rtol=1e-12, atol=1e-14)
