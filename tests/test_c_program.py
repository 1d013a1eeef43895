"""The boundary is a plain C ABI: a C program (tests/c/abi_from_c.c) that
includes only include/ddp_allreduce.h, built with gcc and linked against
the library, plans buckets and exercises the entry points' validation
without PyTorch or Python in the process and without a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gradient_all_reduce_allreduce_amd")
LIB = os.path.join(PKG, "libddp_allreduce.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("libddp_allreduce.so is not built")
    exe = str(tmp_path / "abi_from_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", exe, "-L", PKG,
                    "-lddp_allreduce", "-Wl,-rpath," + PKG], check=True, capture_output=True, text=True)
    p = subprocess.run([exe], capture_output=True, text=True, timeout=60,
                       env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert p.returncode == 0, p.stdout + p.stderr
    assert "all checks passed" in p.stdout
