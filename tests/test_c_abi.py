"""The C ABI from C: include/bpw.h compiles as strict C99 and a C program
linked against libbpw.so runs the host-only entry points (sizes, PQ2 prepare,
refusals, workspace sizes) without a GPU. The program and its expected values
are in tests/c_abi/abi_check.c."""
import os
import shutil
import subprocess

import pytest

import bit_packed_weight_amd as bpw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_c_program_uses_the_abi(tmp_path):
    lib_dir = os.path.dirname(bpw.lib()._name)
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), "-L", lib_dir, "-lbpw",
           f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
