"""The C ABI's host code (argument checks, workspace layouts, tile and grid arithmetic:
csrc/api.hip, csrc/schedule.hip) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer against stub launchers that touch every byte of every extent
they are handed (tests/abi_sanitize_driver.cpp). Runs the argument-error matrix, every
entry point over edge shapes (N = 0, capacity 0 and below N*K, 1024 experts, 64 slots,
more than 2^21 slots) and the size arithmetic at N*K near 2^31 and H = I = 2^20. A
planted one-element overflow must be reported, so the check is known to bite."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_routing_grouped_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("abi") / "abi_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall",
           "-Wno-unused-function", "-I", os.path.join(ROOT, "tests", "abi_stub"),
           "-I", os.path.join(ROOT, "include"), "-x", "c++", os.path.join(CSRC, "api.hip"),
           os.path.join(CSRC, "schedule.hip"), "-x", "none",
           os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return env


def test_abi_host_code_under_sanitizers(driver):
    r = subprocess.run([driver], capture_output=True, text=True, timeout=120, env=_env())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi ok" in r.stdout
    assert "runtime error" not in r.stderr


def test_planted_overflow_is_caught(driver):
    r = subprocess.run([driver, "plant"], capture_output=True, text=True, timeout=120, env=_env())
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr
