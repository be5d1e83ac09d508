"""The C ABI from C: tests/c/abi_host_check.c includes libmoe.h as C99
(gcc, -Wall -Werror), links libmoe.so and exercises the host-side calls
(queries, validation, error strings) without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_is_c99_and_library_links(tmp_path):
    import sparse_mixture_experts_47_amd as m
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "abi_host_check")
    libdir = os.path.dirname(m.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-o", exe,
           m.LIB_PATH, "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ok")
