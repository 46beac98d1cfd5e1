"""The host-side validation of libgdn's C ABI built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; the device code is the normal build) and driven
through every entry point's error paths by a standalone program: no invalid access, no
undefined behaviour, the expected status for every case. No HIP call is made."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_deltanet_linear_prefill_amd")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG),
                    reason="needs the ROCm toolchain")
def test_abi_validation_under_asan_ubsan(tmp_path):
    objs = [os.path.join(PKG, "_build", f"{name}.hip.o")
            for name in ("gdn_chunked", "gdn_scan", "gdn_decode", "gdn_calib")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("build the library first")
    api = tmp_path / "api_san.o"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN_HOST,
                    "-c", os.path.join(PKG, "csrc", "gdn_api.hip"), "-o", str(api)],
                   check=True, capture_output=True, text=True)
    exe = tmp_path / "abi_san"
    subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), str(api), *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi driver ok" in r.stdout
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
