"""The C-ABI boundary from plain C: tests/c_abi/abi_check.c is compiled with gcc as C99
against include/ra.h (no HIP headers), linked against libra.so and run (host-side entry
points only; no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c99_caller(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    import long_context_exact_tiled_amd as m
    if not os.path.exists(m.LIB_PATH):
        from long_context_exact_tiled_amd.build import build
        build()
    libdir = os.path.dirname(m.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "abi_check.c"),
           "-L", libdir, "-l:libra.so", "-Wl,-rpath," + libdir, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert "c abi ok" in out.stdout
