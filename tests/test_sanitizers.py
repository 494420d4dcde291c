"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host routing source (CPU-offloaded routing) and the C oracle are
built with -fsanitize=address,undefined into one test executable
(tests/sanitize/route_check.cpp) that runs both on small seeded inputs and
their degenerate cases; any invalid access, leak or undefined operation aborts
it.  The HIP sources are left out: their device code is not instrumented by
these sanitizers.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(cmd, **kw):
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)


def test_host_routing_and_oracle_under_asan_ubsan(tmp_path):
    if not (shutil.which("gcc") and shutil.which("g++")):
        pytest.skip("gcc/g++ not available")
    obj_o = str(tmp_path / "oracle.o")
    obj_h = str(tmp_path / "host_route.o")
    exe = str(tmp_path / "route_check")
    inc = ["-I", os.path.join(ROOT, "include")]
    steps = [
        ["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-c",
         os.path.join(ROOT, "oracle", "kap_oracle.c"), "-o", obj_o] + SAN,
        ["g++", "-std=c++17", "-pthread", "-c",
         os.path.join(ROOT, "block_sparse_paged_page_amd", "csrc", "host_route.cpp"),
         "-o", obj_h] + inc + SAN,
        ["g++", "-std=c++17", "-pthread", "-fopenmp",
         os.path.join(ROOT, "tests", "sanitize", "route_check.cpp"), obj_h, obj_o, "-o", exe,
         "-lm"] + inc + SAN,
    ]
    for cmd in steps:
        r = _run(cmd)
        if r.returncode != 0 and ("libasan" in r.stdout or "libubsan" in r.stdout):
            pytest.skip("sanitizer runtimes not installed")
        assert r.returncode == 0, r.stdout
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    if r.returncode != 0 and "LeakSanitizer does not work under ptrace" in r.stdout:
        env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
        r = _run([exe], env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "runtime error" not in r.stdout and "ERROR: AddressSanitizer" not in r.stdout, r.stdout
    assert "all checks passed" in r.stdout
