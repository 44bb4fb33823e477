"""The host half of the C ABI (container pack/unpack, PQ2_0 / PTQ1_0
transcodes, sign check, status strings) built with AddressSanitizer and
UndefinedBehaviorSanitizer by g++ and driven by tests/host_sanitize_driver.cpp
on exact-size heap buffers: round trips exact, every documented error
returned, no sanitizer report.  CPU only; needs no HIP runtime."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "hadamard_rotated_quantized_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_abi_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "host_sanitize_driver.cpp"),
           os.path.join(SRC, "tb_host.cpp"), os.path.join(SRC, "tb_blocks_host.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
