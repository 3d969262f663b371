"""The C ABI's argument checks under AddressSanitizer and UndefinedBehaviorSanitizer.

libgsa's sources and tests/sanitize/abi_checks.cpp are built into one host
program with both sanitizers on the host code only (each -fsanitize= after
-Xarch_host; the device code is built as usual and never runs here).  The
program calls every entry point with invalid arguments, sizes up to the int64
extremes, and (without a GPU) valid ones that stop at the device check.  Any
sanitizer report, or a status code other than the documented one, fails.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_softmax_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_checks_under_asan_and_ubsan(tmp_path):
    from gated_softmax_attention_amd.build import SOURCES
    exe = str(tmp_path / "abi_checks")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"),
                                                       "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "abi checks: ok" in r.stdout, out[-4000:]
