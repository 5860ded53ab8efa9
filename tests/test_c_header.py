"""The C ABI from plain C: include/kvss.h compiles as C99 with gcc -Wall -Werror -pedantic, and a
C program linked against libkvss.so gets the documented results from the calls that return
before any HIP call (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

from kv_sparse_speculative_amd import kvss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c_and_links(tmp_path):
    lib_dir = os.path.dirname(kvss.LIB_PATH)
    assert os.path.exists(kvss.LIB_PATH), "build the library first"
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
           "-L" + lib_dir, "-l:libkvss.so", "-Wl,-rpath," + lib_dir, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout
