"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code, gcc).

`oracle_sanitize_driver.c` calls every entry point of the oracle on small seeded
inputs with exactly sized buffers, edge cases included (no rows, every slot
invalid, ids outside [-1,E), repeated experts, K = 1, E = 1, K = E), and checks
the entry points against one another. Built here with the sanitizers, an
out-of-bounds access, a use after free, a leak or undefined behaviour anywhere
in the oracle fails this test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", ORACLE, os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ORACLE, "moe_oracle.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and ("libasan" in r.stderr or "libubsan" in r.stderr):
        pytest.skip("sanitizer runtime not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr, report
    assert r.stdout.strip() == "ok", report
