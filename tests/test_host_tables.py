"""The library's host-side table construction (code levels, thresholds,
bucket search, decode levels), compiled with g++ under the address and
undefined-behaviour sanitizers and checked by tests/host/table_check.cpp.
CPU only: no GPU code is built or run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_quant_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_tables_under_sanitizers(tmp_path):
    exe = str(tmp_path / "table_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(ROOT, "tests", "host", "table_check.cpp"), os.path.join(CSRC, "nf4_table.cpp"),
           "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert run.stdout.strip().endswith("OK")
