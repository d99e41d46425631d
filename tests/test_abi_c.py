"""The C ABI used from plain C99 (gcc, -Wall -Werror, no C++): the header
compiles as C and the validation paths answer as documented.  No GPU."""

import os
import shutil
import subprocess

import pytest

from quantized_kv_top_amd import qsakv

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_client(tmp_path):
    qsakv.lib()                                   # the library is built
    lib_dir = os.path.dirname(qsakv.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi", "abi_check.c"), "-L", lib_dir, "-lqsakv",
           "-Wl,-rpath," + lib_dir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
