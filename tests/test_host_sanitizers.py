"""The planner and the C-ABI validation layer under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/host_sanitize/host_check.cpp is built with g++ together with csrc/plan.cpp and
csrc/mla_api.cpp (no kernels: their launchers are stubs that abort) and run over a few hundred
random problems (batch up to 1,200, lengths up to 2^20, every page size and row count, forced
split counts, 1 to 1,024 compute units) plus every validation path.  Any out-of-bounds access,
leak of the host plan, signed overflow or misaligned access ends the run with an error."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_decode_attention_paged_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_planner_and_validation_under_asan_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("needs g++ and the HIP headers")
    exe = tmp_path / "host_check"
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-Wall", *sanitize, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_sanitize", "host_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "mla_api.cpp"), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe), "400"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:], r.stderr[-4000:])
