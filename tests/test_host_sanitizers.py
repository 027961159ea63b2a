"""The C-ABI front end (api.cpp, plan.cpp: plain C++, no HIP) built with
AddressSanitizer and UndefinedBehaviorSanitizer, then tests/test_abi.py run
against that build in a child process (sanitizer runtimes preloaded). Every
validation path of the ABI tests executes under the sanitizers; any report
fails the child, and so this test. CPU only: the launchers are stand-ins that
report a launch failure (tests/sanitize/host_stubs.cpp).
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_87_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_validation_under_asan_and_ubsan():
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not available")
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libssm_scan_host_sanitized.so")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp")]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
             "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    r = subprocess.run(["g++", *flags, *srcs, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["SSM_SCAN_LIBRARY"] = lib
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        "-k", "not bench_refuses and not header_is_plain"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
