"""The C ABI from plain C: tests/c_abi_check.c compiled as C99 with gcc against include/mla.h
and linked to libmla.so, then run (host-only calls; CPU)."""
import os
import shutil
import subprocess

import pytest

from mla_decode_attention_paged_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_compiles_as_c_and_host_calls_behave(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = B.lib()   # builds nothing; fails loudly if libmla.so is missing
    lib_path = lib._name
    exe = tmp_path / "c_abi_check"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), lib_path, "-o", str(exe),
           "-Wl,-rpath," + os.path.dirname(lib_path)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr[-2000:])
