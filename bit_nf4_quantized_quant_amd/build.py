"""Build libqlora.so in-tree with hipcc for gfx950.

Usage: python -m bit_nf4_quantized_quant_amd.build  (or call build_library()).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libqlora.so")

SOURCES = ["api.hip", "quant.hip", "decode.hip", "gemv.hip", "gemm.hip", "nf4_table.cpp"]

# -ffp-contract=off: the dequantization arithmetic is specified as separate
# fp32 roundings; fused multiply-adds are written explicitly where wanted.
# Packed fp32 instructions are disabled on the device.  The atomic optimizer
# is off: every device atomic here is issued by one lane, and the optimizer's
# wave-wide rewrite waits for each reply as soon as it is issued.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the QLoRA library needs ROCm's hipcc to build")


# Per-source flags.  gemv.hip, decode.hip: the decode kernels' leading pointer
# and size arguments are preloaded into scalar registers at dispatch (gfx950
# kernarg preloading), so their first loads do not wait for a kernel-argument
# fetch.
_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
SOURCE_FLAGS = {"gemv.hip": _PRELOAD, "decode.hip": _PRELOAD, "gemm.hip": _PRELOAD}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + FLAGS + SOURCE_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    return obj


CALIB_SOURCE = "calib.hip"
CALIB_PATH = os.path.join(PKG, "libqlora_calib.so")


def build_calib(verbose: bool = False) -> str:
    """The benchmark's reference kernels (empty kernel, plain streaming read),
    linked separately from the layer's library as libqlora_calib.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = _compile(CALIB_SOURCE, verbose)
    tmp = CALIB_PATH + ".tmp"
    res = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", obj, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, CALIB_PATH)
    return CALIB_PATH


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libqlora.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    print(build_calib(verbose="-v" in sys.argv))
