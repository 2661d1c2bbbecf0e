"""Host check of the kernels' memory index arithmetic (no GPU).

tests/c/index_check.cpp calls the index functions the kernels themselves call
(chunked_linear_recurrence_amd/csrc/ssd_index.h: the x, b_in, cum, dblk and B-tile copies
of chunk_scan, its staged output stores, and the state tile order of state_pass) for
every compiled shape, wave, lane and item, and checks every global read against its row
or tile, every LDS access against its region, and that each tile is covered exactly
once.  It also plants the per-wave guard that once let lanes past a decay row shorter than
a wave (chunk lengths below 256) and requires the check to reject it."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

C_DIR = os.path.join(ROOT, "tests", "c")


def _hipcc():
    return os.path.exists(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")) or shutil.which("hipcc")


def test_kernel_index_functions_stay_in_bounds():
    if not _hipcc():
        pytest.skip("hipcc not available")
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_build", os.path.join(C_DIR, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build_index_check()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures: 0" in r.stdout
    assert "planted per-wave guard detected: yes" in r.stdout
