"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The C ABI's argument checks, the page pool (free list, reference counts, copy-on-write
decisions) and the slot scheduler are built with host-side ASan + UBSan into a test
library (``build.build_asan``: only those sources instrumented, any error fatal), and the
CPU tests that drive them -- ``test_abi_cpu.py`` and ``test_sched_cpu.py`` -- run against
it in a child process that preloads the sanitizer runtime.  Any sanitizer report fails
the test."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_is_clean_under_asan_and_ubsan():
    from paged_kv_attention_31_amd import build as B

    kernel_objs = [os.path.join(B.BUILD, os.path.splitext(x)[0] + ".o") for x in B.SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs + [B.LIB_PATH]):
        try:
            B.build()
        except RuntimeError as e:
            pytest.skip(f"library build unavailable: {e}")
    try:
        lib = B.build_asan()
        rt = B.asan_runtime()
    except RuntimeError as e:  # no ROCm toolchain on this host
        pytest.skip(f"sanitizer build unavailable: {e}")
    env = dict(os.environ)
    env["PAGEDATTN_LIB"] = lib
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # CPython's own allocations are not the subject: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"),
           os.path.join(ROOT, "tests", "test_sched_cpu.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
    # the child really loaded the sanitized build, with the runtime in place, and the build
    # carries the instrumentation
    probe = subprocess.run(
        [sys.executable, "-c",
         "from paged_kv_attention_31_amd import _lib; _lib.load(); print(_lib.LIB_PATH); "
         "m = open('/proc/self/maps').read(); "
         "print('asan-rt' if 'libclang_rt.asan' in m else 'no-rt', "
         "'lib' if _lib.LIB_PATH in m else 'no-lib')"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.stdout.split() == [lib, "asan-rt", "lib"], probe.stdout + probe.stderr
    with open(lib, "rb") as f:
        assert b"__asan_report_store" in f.read()
