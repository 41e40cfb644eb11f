"""The C ABI from plain C: tests/abi_check.c is compiled as C99 against
include/flint_attn.h, linked to the built library and run (host-side
contract only: sizes, argument checks before any launch, status strings)."""

import os
import shutil
import subprocess

import pytest

import attention_head_rmsnorm_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_against_the_header(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = fa.library_path()
    libdir = os.path.dirname(lib)
    exe = tmp_path / "abi_check"
    build = subprocess.run(
        [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "tests", "abi_check.c"), lib, f"-Wl,-rpath,{libdir}", "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failed" in run.stdout
