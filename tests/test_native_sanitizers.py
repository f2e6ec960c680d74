"""The host library under AddressSanitizer and UBSan (CPU, g++ only).

Builds tests/native/alloc_fuzz.cpp together with every host source (no GPU
code): allocator, plans, staging, scheduler, hybrid manager, utilisation;
runs seeded random operations with invariant checks.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_kv_cache_257_amd", "csrc", "host")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_allocator_fuzz_under_sanitizers(tmp_path):
    exe = str(tmp_path / "alloc_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "alloc_fuzz.cpp"),
           *[os.path.join(SRC, f) for f in ("pool.cpp", "plan.cpp", "plan_shared.cpp", "prepare.cpp", "prefill_plan.cpp",
                                            "utilisation.cpp", "hybrid.cpp", "sched.cpp")], "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "12"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "alloc_fuzz ok" in r.stdout
