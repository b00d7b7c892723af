"""The C ABI from plain C: tests/c/c_client.c, a C99 program that includes
include/tea.h and links libtea.so, is compiled with gcc (-std=c99 -pedantic,
warnings as errors) and run on the CPU.  It calls every entry point on
arguments answered before any HIP call (validation, workspace sizes, status
strings), so the header is checked as C (not only C++) and the exported
symbols as linkable."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "tiled_exact_attention_amd")
LIB = os.path.join(LIB_DIR, "libtea.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.skipif(not os.path.exists(LIB), reason="libtea.so not built")
def test_c_client(tmp_path):
    exe = tmp_path / "c_client"
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "c_client.c"), "-L", LIB_DIR, "-ltea",
                    f"-Wl,-rpath,{LIB_DIR}", "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "c client ok" in r.stdout
