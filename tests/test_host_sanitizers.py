"""The C ABI's host-side validation and planning (api.hip, plan.hip) built as
plain host C++ with AddressSanitizer and UndefinedBehaviorSanitizer, kernel
launchers stubbed, and driven through every entry point's error paths,
accepted paths and extreme sizes (tests/host_asan/harness.cpp). CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS = os.path.join(ROOT, "tests", "host_asan", "harness.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_validation_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "harness"
    flags = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include"), "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run(["g++", *flags, HARNESS, "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0"))
    assert r.returncode == 0 and r.stdout.strip().endswith("harness ok"), r.stdout + r.stderr
