"""Host-side checks of the kernels' LDS layouts and element masks (no GPU).

Compiles ``tests/host/layout_check.cpp`` -- which includes the kernels' own
index helpers -- for the host and runs it: every MFMA operand read from LDS
(16-byte row reads and gfx950 transposing reads) must deliver exactly the
logical elements its K slots stand for, without LDS bank conflicts.
``tests/host/mask_check.cpp`` checks that the range masks' one-run form,
as the tile steps evaluate it, agrees with the kernels' visibility predicate.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_host_check(tmp_path, name):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / name)
    src = os.path.join(ROOT, "tests", "host", name + ".cpp")
    r = subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17", src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout


def test_lds_layouts(tmp_path):
    run_host_check(tmp_path, "layout_check")


def test_range_mask_runs(tmp_path):
    run_host_check(tmp_path, "mask_check")
