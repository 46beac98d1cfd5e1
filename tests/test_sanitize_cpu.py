"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code
only, gcc) and driven over several shapes, a head subset, several thread counts and rejected
arguments: no invalid access, no undefined behaviour, the same bits for any thread count."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver ok" in r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
