"""Host-side checks of the kernels' LDS tile layouts (no GPU).

Builds tests/layout_check.cpp with g++ against the kernels' own layout
header and runs it: bijection and inverse of the row-group layout, the
address steps the kernels rely on, the matrix-core operand elements that a
simulated transpose read delivers, the producer / consumer agreement on the
P^T / dS^T tile, and freedom from LDS bank conflicts.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "io_aware_tiled_fa_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_lds_layouts(tmp_path):
    exe = str(tmp_path / "layout_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC, os.path.join(HERE, "layout_check.cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all layout checks passed" in r.stdout
