"""The public header compiles as strict C99 and a plain-C client links against libsage_fp4.so and
gets the documented results from every entry point that needs no GPU (tests/c_abi_check.c)."""
import os
import shutil
import subprocess

import pytest

from bit_attention_amd import binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_client(tmp_path):
    libdir = os.path.dirname(bnd.LIB_PATH)
    exe = tmp_path / "c_abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
           "-L", libdir, "-lsage_fp4", f"-Wl,-rpath,{libdir}", "-Wl,--allow-shlib-undefined", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "C ABI OK" in r.stdout
