"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the sanitizer variants of the oracle (oracle.c) and of libtcm's host
code (tcm_api.cpp: the C ABI's validation, planning and dispatch; the device
objects are the ordinary ones and are never launched here), then runs the
oracle's pins and the C-ABI tests against them in a child process with the
sanitizer runtimes preloaded.  Any sanitizer report fails the child.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_code_clean_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    from oracle import oracle as orc
    from tensor_core_matrix_amd import build as tcm_build

    san_lib = tcm_build.build_sanitized(verbose=False)
    san_oracle = orc.build(force=True, sanitize=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{asan}:{ubsan}",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "TCM_LIBRARY": san_lib,
        "ORACLE_LIBRARY": san_oracle,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_oracle.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
