"""The C ABI from a plain C program (tests/c/abi_layer.c): the header is valid C, and one
layer run through ssd_chunk_scan_fwd from C (device buffers from the HIP runtime) matches
the fp64 oracle.  The program is built by __graft_entry__.build() (tests/c/build.py)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "tests", "c", "abi_layer.c")
BIN = os.path.join(ROOT, "tests", "c", "_build", "abi_layer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_header_and_caller_compile_as_c():
    if shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM, "include")):
        pytest.skip("gcc or the ROCm headers are not available")
    r = subprocess.run(["gcc", "-fsyntax-only", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.gpu
def test_layer_from_c_matches_oracle():
    if not os.path.exists(BIN):
        pytest.skip("tests/c/_build/abi_layer not built (run __graft_entry__.build())")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "y err" in r.stdout
