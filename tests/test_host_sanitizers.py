"""The library's host code (launch plans, workspace sizes, argument checks) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: api.hip is compiled with
the sanitizers on its host side only (the device code is the normal build), linked
with the other objects into a driver that calls every host path that returns before
a launch (tests/sanitize/host_checks.cpp), and run."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "speculative_decoding_verify_amd")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_paths_under_address_and_undefined_behaviour_sanitizers():
    from speculative_decoding_verify_amd import build as b
    objdir = os.path.join(PKG, "_build")
    others = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in b.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        b.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory() as tmp:
        api_o = os.path.join(tmp, "api.o")
        r = subprocess.run(flags + san + ["-c", "-o", api_o, os.path.join(PKG, "csrc", "api.hip")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        syms = subprocess.run(["nm", api_o], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms    # the host code is instrumented
        drv_o = os.path.join(tmp, "host_checks.o")
        r = subprocess.run(flags + san + ["-c", "-o", drv_o, os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        exe = os.path.join(tmp, "host_checks")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", "-o", exe, drv_o, api_o]
                           + others, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and "host checks ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
