"""The library's exact mean of the block constants (exact_mean.h: mantissa
sums per exponent, one multi-word integer, one rounding to fp32), compiled
with g++ for the host and checked against the oracle's mean (the exact
rational mean rounded once to fp32) on seeded inputs: typical NF4 block
maxima, values spread over the whole fp32 range including subnormals,
exact rounding ties, and a few degenerate cases.  CPU only."""

import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_quant_amd", "csrc")


def cases():
    rng = np.random.default_rng(2024)
    out = []
    for n in (1, 2, 3, 64, 255, 256, 257, 4096, 65536):   # |N(0, 0.02)| block maxima
        out.append(np.abs(rng.normal(0, 0.02, (n, 64))).max(axis=1).astype(np.float32))
    for n in (1, 7, 100, 1000, 50000):                    # any positive fp32, subnormals included
        bits = rng.integers(1, 0x7F800000, n, dtype=np.int64).astype(np.uint32)
        out.append(bits.view(np.float32))
    for n in (2, 5, 33):                                  # one exponent band, many mantissas
        out.append((1.0 + rng.integers(0, 1 << 23, n) / float(1 << 23)).astype(np.float32))
    one = np.float32(1.0)
    out.append(np.array([one, np.nextafter(one, np.float32(2))], np.float32))      # mean at a tie: rounds to even
    out.append(np.array([np.nextafter(one, np.float32(2)), np.nextafter(np.nextafter(one, np.float32(2)),
                                                                        np.float32(2))], np.float32))
    out.append(np.zeros(10, np.float32))                                          # all zero
    out.append(np.array([np.float32(1e-45)] * 3, np.float32))                     # smallest subnormal
    out.append(np.array([np.float32(1e-45), 0, 0], np.float32))                   # below half an ulp of 0
    out.append(np.array([np.finfo(np.float32).max] * 4, np.float32))              # largest finite
    out.append(np.array([np.finfo(np.float32).max, np.float32(1e-45)], np.float32))
    return out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_exact_mean_matches_oracle(tmp_path):
    exe = str(tmp_path / "mean_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", CSRC, os.path.join(ROOT, "tests", "host", "mean_check.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    data = cases()
    path = str(tmp_path / "values.bin")
    with open(path, "wb") as f:
        for v in data:
            f.write(struct.pack("<Q", v.size))
            f.write(np.ascontiguousarray(v, np.float32).tobytes())
    run = subprocess.run([exe, path], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr[-2000:]
    got = [int(x, 16) for x in run.stdout.split()]
    assert len(got) == len(data)
    for i, v in enumerate(data):
        want = int(np.float32(oracle.mean_f32(v)).view(np.uint32))
        assert got[i] == want, f"case {i} (n={v.size}): library {got[i]:08x}, oracle {want:08x}"
