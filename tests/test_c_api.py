"""The C ABI from C: a C99 program compiled with gcc against include/lvsa.h and
linked to liblvsa.so (no Python in the calls).  CPU only: it builds and checks
masks and argument errors that return before any device work."""

import os
import shutil
import subprocess

import pytest

import block_sparse_attention_lvsa_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_uses_the_abi(tmp_path):
    L.library()  # the shared library must be built
    lib_dir = os.path.dirname(L.LIB_PATH)
    exe = tmp_path / "abi_demo"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_api", "abi_demo.c"), "-o", str(exe),
           "-L", lib_dir, "-llvsa", f"-Wl,-rpath,{lib_dir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
