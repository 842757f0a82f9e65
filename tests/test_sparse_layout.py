"""Host logic of the bf16 forward's structured-sparse operand (kan_sparse.h):
the column order and the per-span table, checked for every (K, base) the
planner accepts for the sparse form by a C++ program built with the host
compiler.  Plain integer logic; no GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "kolmogorov_arnold_network_amd", "csrc")


def test_sparse_column_order_and_table(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "sparse_layout_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, os.path.join(HERE, "host", "sparse_layout_check.cpp"),
                    "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    cases = int(out.stdout.split()[1])
    assert cases >= 40, out.stdout     # every NG (4, 6, 8) with and without a base branch
    assert "mismatches 0" in out.stdout
