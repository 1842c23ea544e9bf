"""QLoRA NF4 quantized linear layer on AMD MI355X (gfx950).

The compute lives in libqlora.so (hand-written HIP kernels behind the C ABI in
include/qlora.h).  This package only binds it: ``_lib`` mirrors the C entry
points one to one, and the helpers below allocate output tensors with torch
and pass them through.  Nothing here computes any part of the layer.
"""

from __future__ import annotations

import dataclasses

from . import _lib
from ._lib import (QLoraError, lib, qlora_double_quant, qlora_double_quant_workspace,  # noqa: F401
                   qlora_linear_bwd, qlora_linear_bwd_workspace, qlora_linear_fwd,
                   qlora_linear_fwd_wait_counter_offset, qlora_linear_fwd_workspace, qlora_merge,
                   qlora_nf4_dequant, qlora_nf4_levels,
                   qlora_nf4_quantize, qlora_nf4_quantize_bf16, qlora_nf4_sizes)


@dataclasses.dataclass
class QuantizedWeight:
    """A frozen NF4 weight [N, K] with double-quantized constants (device tensors)."""
    N: int
    K: int
    codes: "object"   # uint8 [N, K/2]
    absmax: "object"  # fp32 [N*K/64] (first-level constants, kept for inspection)
    c2: "object"      # uint8 [N*K/64]
    c1: "object"      # fp32 [ceil(N*K/16384)]
    mean: "object"    # fp32 [1]
    table: int = 0    # code table: 0 NF4, 1 uniform 4-bit, 2 FP4


def quantize(W, stream=None, table: int = 0) -> QuantizedWeight:
    """NF4-quantize an fp32 or bf16 [N, K] device tensor and double-quantize its constants."""
    import torch
    N, K = W.shape
    code_bytes, n_c2, n_c1 = qlora_nf4_sizes(N, K)
    dev = W.device
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    absmax = torch.empty(n_c2, dtype=torch.float32, device=dev)
    c2 = torch.empty(n_c2, dtype=torch.uint8, device=dev)
    c1 = torch.empty(max(n_c1, 1), dtype=torch.float32, device=dev)
    mean = torch.zeros(1, dtype=torch.float32, device=dev)
    if W.dtype == torch.bfloat16:
        qlora_nf4_quantize_bf16(W, codes, absmax, stream, table)
    else:
        qlora_nf4_quantize(W, codes, absmax, stream, table)
    ws = torch.empty(max(qlora_double_quant_workspace(n_c2), 8), dtype=torch.uint8, device=dev)
    qlora_double_quant(absmax, c2, c1, mean, ws, stream)
    return QuantizedWeight(N, K, codes, absmax, c2, c1, mean, table)


def save_quantized(q: QuantizedWeight, path: str) -> None:
    """Write a quantized weight (codes, constants, mean, shape, table) to an
    uncompressed .npz file; plain arrays only, nothing pickled."""
    import numpy as np

    def arr(t):
        return None if t is None else t.detach().cpu().numpy()
    fields = {"N": np.int64(q.N), "K": np.int64(q.K), "table": np.int64(q.table), "codes": arr(q.codes),
              "c2": arr(q.c2), "c1": arr(q.c1), "mean": arr(q.mean)}
    if q.absmax is not None:
        fields["absmax"] = arr(q.absmax)
    np.savez(path, **fields)


def load_quantized(path: str, device="cuda") -> QuantizedWeight:
    """Read a weight written by save_quantized onto `device` (no pickle)."""
    import numpy as np
    import torch
    with np.load(path, allow_pickle=False) as z:
        N, K, table = int(z["N"]), int(z["K"]), int(z["table"])
        code_bytes, n_c2, n_c1 = qlora_nf4_sizes(N, K)
        codes, c2, c1, mean = z["codes"], z["c2"], z["c1"], z["mean"]
        if (codes.dtype != np.uint8 or codes.shape != (N, K // 2) or c2.dtype != np.uint8 or c2.shape != (n_c2,)
                or c1.dtype != np.float32 or c1.size < max(n_c1, 1) or mean.dtype != np.float32
                or mean.shape != (1,) or table not in (0, 1, 2)):
            raise ValueError(f"{path}: not a quantized [{N}, {K}] weight")
        absmax = torch.from_numpy(z["absmax"]).to(device) if "absmax" in z.files else None
        return QuantizedWeight(N, K, torch.from_numpy(codes).to(device), absmax, torch.from_numpy(c2).to(device),
                               torch.from_numpy(c1).to(device), torch.from_numpy(mean).to(device), table)


def dequantize(q: QuantizedWeight, stream=None):
    """bf16 [N, K] weight (returned as int16 bit patterns viewed as bfloat16)."""
    import torch
    out = torch.empty((q.N, q.K), dtype=torch.bfloat16, device=q.codes.device)
    qlora_nf4_dequant(q.codes, q.c2, q.c1, q.mean, q.N, q.K, out, stream, q.table)
    return out


def merge(q: QuantizedWeight, A, B, alpha: float, stream=None):
    """The merged bf16 weight W_deq + (alpha / r) B A, [N, K]."""
    import torch
    out = torch.empty((q.N, q.K), dtype=torch.bfloat16, device=q.codes.device)
    qlora_merge(q.codes, q.c2, q.c1, q.mean, q.N, q.K, A, B, alpha, out, stream, q.table)
    return out


def fwd_workspace(M: int, N: int, K: int, r: int, device):
    """A forward workspace, zero-filled as the library requires before its first
    use.  The kernels keep launch counters and partial sums in it between calls,
    so after a call it is not zero: reuse it as it is (any shapes it is large
    enough for), and do not write to it except to clear the wait counter."""
    import torch
    n = max(qlora_linear_fwd_workspace(M, N, K, r), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def fwd_wait_count(workspace) -> int:
    """The forward workspace's wait counter (qlora_linear_fwd_wait_counter_offset):
    how many values decode-size launches (M <= 16) computed themselves after a
    wait for another workgroup's partial result (a part of H, or a K slice's
    partial product) gave up.  Results stay correct either way; nonzero means
    the slow fallback ran.  Synchronizes with the device (the read is a
    device-to-host copy)."""
    import torch
    off = qlora_linear_fwd_wait_counter_offset()
    return int(workspace[off:off + 4].view(torch.int32).item())


def clear_fwd_wait_count(workspace) -> None:
    """Zero the forward workspace's wait counter (a 4-byte fill on the current stream)."""
    off = qlora_linear_fwd_wait_counter_offset()
    workspace[off:off + 4].zero_()


def linear_fwd(X, q: QuantizedWeight, A, B, alpha: float, workspace=None, want_h: bool = True, stream=None):
    """Y = X W_deq^T + (alpha/r) (X A^T) B^T.  X, A, B bf16; returns (Y bf16 [M,N], H fp32 [M,r] or None).

    A = B = None means no adapter (r = 0): Y = X W_deq^T."""
    import torch
    M = X.shape[0]
    r = 0 if A is None else A.shape[0]
    Y = torch.empty((M, q.N), dtype=torch.bfloat16, device=X.device)
    H = torch.empty((M, r), dtype=torch.float32, device=X.device) if want_h and r > 0 else None
    if workspace is None:
        workspace = fwd_workspace(M, q.N, q.K, r, X.device)
    qlora_linear_fwd(X, q.codes, q.c2, q.c1, q.mean, A, B, alpha, Y, H, workspace, q.N, stream, q.table)
    return Y, H


def linear_bwd(dY, X, q: QuantizedWeight, A, B, alpha: float, H=None, want_dx: bool = True, stream=None):
    """Gradients (dX or None, dA, dB) of the QLoRA linear; the NF4 weight gets none.

    A = B = None means no adapter (r = 0): only dX, and dA = dB = None."""
    import torch
    M, K = X.shape
    r = 0 if A is None else A.shape[0]
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=X.device) if want_dx else None
    dA = torch.empty((r, K), dtype=torch.bfloat16, device=X.device) if r > 0 else None
    dB = torch.empty((q.N, r), dtype=torch.bfloat16, device=X.device) if r > 0 else None
    ws = torch.empty(max(qlora_linear_bwd_workspace(M, q.N, K, r), 256), dtype=torch.uint8, device=X.device)
    qlora_linear_bwd(dY, X, q.codes, q.c2, q.c1, q.mean, A, B, alpha, H, dX, dA, dB, ws, stream, q.table)
    return dX, dA, dB
