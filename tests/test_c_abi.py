"""The C-ABI from a plain C program (no Python, no torch): tests/c_abi/check.c is built
with gcc against include/int8attn.h and libint8attn.so and run; it checks the version and
the documented error codes of rejected calls (no GPU needed: nothing reaches the device)."""
import os
import shutil
import subprocess

import pytest

import int8_kv_cache_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_caller(tmp_path):
    lib_dir = os.path.dirname(m.LIB_PATH)
    exe = tmp_path / "check"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "check.c"), "-L", lib_dir, "-lint8attn",
                    "-Wl,-rpath," + lib_dir, "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c-abi ok" in res.stdout
