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


def test_c_program_under_host_sanitizers(tmp_path):
    """The same program against a build of the library whose host code carries
    AddressSanitizer and UndefinedBehaviorSanitizer (device code is built as
    usual; the sanitizers apply to the host side only): every validation path
    runs without a memory error or undefined behaviour."""
    from attention_head_rmsnorm_amd import build as b

    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("no ROCm clang")
    lib = tmp_path / "libflint_attn_san.so"
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-O3",)] + [
        "-O1", "-g",
        "-Xarch_host", "-fsanitize=address",
        "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-omit-frame-pointer"]
    res = subprocess.run([b.hipcc(), *flags, "-I", b.INCLUDE, *b.SRCS, "-o", str(lib)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    exe = tmp_path / "abi_check_san"
    res = subprocess.run([clang, "-std=c99", "-g", "-fsanitize=address,undefined", "-I",
                          os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_check.c"),
                          str(lib), f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failed" in run.stdout
