"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

This module only draws random numbers and stores them in the storage types
the layer consumes (fp32 weights, bf16 activations and LoRA factors).  It holds
none of the layer's own arithmetic, so both the CPU oracle and the GPU library
can be fed from it without sharing any of the method's code.

Distributions follow the workloads on the pages: base weights ~N(0, 0.02)
(the itwiki "QLoRA" page, NF4 section, draws its example weights this way with
seed 0), activations and upstream gradients ~N(0, 1), LoRA factors A with
standard deviation 1/K and B with standard deviation 0.01.  The second argument
of N(., .) is read as a standard deviation throughout, as numpy's
``normal(loc, scale)`` does.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np

# Seeds per tensor role: W uses seed 0 as in the pages' worked example.
SEED_W, SEED_X, SEED_A, SEED_B, SEED_DY = 0, 1, 2, 3, 4

_CHUNK = 1 << 22  # elements per independent sub-stream (and per worker task)
_WORKERS = min(16, os.cpu_count() or 1)


def normal_f32(seed, shape, std: float) -> np.ndarray:
    """fp64 normal draws rounded to fp32 (round to nearest even).

    Element i belongs to chunk i // 2^22; chunk c is drawn from the PCG64
    stream of ``seed`` advanced by c jumps, so chunks are independent and are
    filled in parallel.  A tensor of at most one chunk is exactly the first
    ``count`` draws of ``np.random.default_rng(seed).normal(0, std)``.
    """
    count = int(np.prod(shape))
    out = np.empty(count, dtype=np.float32)
    nchunks = -(-count // _CHUNK)
    base = np.random.PCG64(seed)

    def fill(c):
        n = min(_CHUNK, count - c * _CHUNK)
        rng = np.random.Generator(base.jumped(c) if c else np.random.PCG64(seed))
        out[c * _CHUNK:c * _CHUNK + n] = rng.normal(0.0, std, size=n)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with concurrent.futures.ThreadPoolExecutor(min(_WORKERS, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store fp32 values as bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite (so the 32-bit sum below cannot wrap); this is only the
    storage conversion of synthetic data.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = u + np.uint32(0x7FFF)
    out += (u >> 16) & np.uint32(1)
    out >>= 16
    return out.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed, shape, std: float) -> np.ndarray:
    """fp64 normal draws -> fp32 -> bf16 bits (uint16)."""
    return f32_to_bf16_bits(normal_f32(seed, shape, std))


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    M: int
    N: int
    K: int
    r: int
    alpha: float = 16.0
    seed_offset: int = 0


def make_layer(shape: LayerShape, with_dy: bool = False) -> dict:
    """All inputs of one QLoRA linear: W fp32 [N,K], X/A/B (and dY) as bf16 bits."""
    def seed(role):
        # standard workloads use the plain role seeds; decoder layers key a
        # seed sequence on (layer/module seed, role)
        return role if shape.seed_offset == 0 else [shape.seed_offset, role]
    d = {
        "W": normal_f32(seed(SEED_W), (shape.N, shape.K), 0.02),
        "X": normal_bf16(seed(SEED_X), (shape.M, shape.K), 1.0),
        "A": normal_bf16(seed(SEED_A), (shape.r, shape.K), 1.0 / shape.K),
        "B": normal_bf16(seed(SEED_B), (shape.N, shape.r), 0.01),
    }
    if with_dy:
        d["dY"] = normal_bf16(seed(SEED_DY), (shape.M, shape.N), 1.0)
    return d


# The workloads: a small single layer, a 4096x4096 decode GEMV, Llama-7B-shaped
# MLP projections, a 65B-scale training layer and a whole 7B-shaped decoder.
SINGLE = LayerShape("single_256x256_m16", M=16, N=256, K=256, r=8)
DECODE = [LayerShape(f"decode_4096x4096_m{m}", M=m, N=4096, K=4096, r=64) for m in (1, 4, 16)]
MLP = [LayerShape(f"mlp_{nm}_m{m}", M=m, N=n, K=k, r=64)
       for m in (1, 16, 256)
       for nm, n, k in (("gate_up_11008x4096", 11008, 4096), ("down_4096x11008", 4096, 11008))]
TRAIN65B = LayerShape("train65b_22016x8192_m4096", M=4096, N=22016, K=8192, r=64)

# 7B-shaped decoder: (module name, N, K, LoRA rank or 0)
DECODER_MODULES = (("q", 4096, 4096, 16), ("k", 4096, 4096, 0), ("v", 4096, 4096, 16),
                   ("o", 4096, 4096, 0), ("gate", 11008, 4096, 0), ("up", 11008, 4096, 0),
                   ("down", 4096, 11008, 0))
DECODER_LAYERS = 32


def decoder_seed(layer: int, module: int) -> int:
    return 1000 + 10 * layer + module


# The same decoder with the linears that read the same input concatenated
# along N (q|k|v and gate|up): one quantized weight and one launch per group.
# The q and v adapters (r = 16 each) become one rank-32 adapter of the group:
# A stacks A_q over A_v, and B is block-structured -- q's rows use columns
# 0..15, v's rows columns 16..31, k's rows are zero -- with alpha = 32 so that
# alpha / r stays 1.
DECODER_FUSED = (("qkv", 12288, 4096, 32), ("o", 4096, 4096, 0), ("gate_up", 22016, 4096, 0),
                 ("down", 4096, 11008, 0))
FUSED_QKV_ALPHA = 32.0


def fused_qkv_b_mask(N: int = 12288, r: int = 32) -> np.ndarray:
    """Where the fused q|k|v adapter's B [N, r] may be non-zero (bool)."""
    seg = N // 3
    mask = np.zeros((N, r), dtype=bool)
    mask[:seg, : r // 2] = True          # q rows: q's 16 adapter columns
    mask[2 * seg:, r // 2:] = True       # v rows: v's 16 adapter columns
    return mask
