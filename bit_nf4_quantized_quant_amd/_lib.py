"""ctypes binding of libqlora.so (the C ABI declared in include/qlora.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers, sizes and the current HIP stream
to the library, and raises QLoraError on a non-zero status.  There is no
fallback: if libqlora.so is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

QLORA_OK, QLORA_EINVAL, QLORA_ESHAPE, QLORA_EHIP = 0, 1, 2, 3

_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_int = ctypes.c_int
_p = ctypes.c_void_p
_f = ctypes.c_float

# name -> (restype, argtypes), mirroring include/qlora.h
SIGNATURES = {
    "qlora_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_nf4_sizes": (ctypes.c_int, [_i64, _i64, _p, _p, _p]),
    "qlora_nf4_levels": (ctypes.c_int, [_int, _p]),
    "qlora_nf4_quantize": (ctypes.c_int, [_p, _i64, _i64, _int, _p, _p, _p]),
    "qlora_nf4_quantize_bf16": (ctypes.c_int, [_p, _i64, _i64, _int, _p, _p, _p]),
    "qlora_double_quant_workspace": (_sz, [_i64]),
    "qlora_double_quant": (ctypes.c_int, [_p, _i64, _p, _p, _p, _p, _sz, _p]),
    "qlora_nf4_dequant": (ctypes.c_int, [_p, _p, _p, _p, _int, _i64, _i64, _p, _p]),
    "qlora_merge": (ctypes.c_int, [_p, _p, _p, _p, _int, _i64, _i64, _p, _p, _i64, _f, _p, _p]),
    "qlora_linear_fwd_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "qlora_linear_fwd": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _int, _p, _p, _i64, _f, _p,
                                        _p, _p, _sz, _p]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _int, _p, _p, _i64, _f,
                                                _p, _p, _p]),
    "qlora_linear_fwd_wait_counter_offset": (_sz, []),
    "qlora_linear_bwd_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "qlora_linear_bwd": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _int, _p, _p, _i64, _f,
                                        _p, _p, _p, _p, _p, _sz, _p]),
}


class QLoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqlora.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqlora.so is not built ({LIB_PATH}); run "
                              "`python -m bit_nf4_quantized_quant_amd.build` (needs hipcc)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().qlora_status_str(status).decode()


def _check(status: int, where: str) -> None:
    if status != QLORA_OK:
        raise QLoraError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libqlora works on GPU tensors only")


# ---------------------------------------------------------------- the C ABI, by name

def qlora_nf4_sizes(N: int, K: int):
    cb, n2, n1 = _i64(), _i64(), _i64()
    _check(lib().qlora_nf4_sizes(N, K, ctypes.byref(cb), ctypes.byref(n2), ctypes.byref(n1)), "qlora_nf4_sizes")
    return cb.value, n2.value, n1.value


def qlora_nf4_levels(table: int = 0):
    buf = (ctypes.c_float * 16)()
    _check(lib().qlora_nf4_levels(table, buf), "qlora_nf4_levels")
    return list(buf)


def qlora_nf4_quantize(W, codes, absmax, stream=None, table: int = 0):
    _need_cuda(W, codes, absmax)
    N, K = W.shape
    _check(lib().qlora_nf4_quantize(_ptr(W), N, K, table, _ptr(codes), _ptr(absmax), _stream(stream)),
           "qlora_nf4_quantize")


def qlora_nf4_quantize_bf16(W, codes, absmax, stream=None, table: int = 0):
    """W: a bf16 (or int16 bit-pattern) [N, K] device tensor."""
    _need_cuda(W, codes, absmax)
    N, K = W.shape
    _check(lib().qlora_nf4_quantize_bf16(_ptr(W), N, K, table, _ptr(codes), _ptr(absmax), _stream(stream)),
           "qlora_nf4_quantize_bf16")


def qlora_double_quant_workspace(n_c2: int) -> int:
    return lib().qlora_double_quant_workspace(n_c2)


def qlora_double_quant(absmax, c2, c1, mean, workspace, stream=None):
    _need_cuda(absmax, c2, c1, mean, workspace)
    _check(lib().qlora_double_quant(_ptr(absmax), absmax.numel(), _ptr(c2), _ptr(c1), _ptr(mean),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "qlora_double_quant")


def qlora_nf4_dequant(codes, c2, c1, mean, N: int, K: int, W_bf16, stream=None, table: int = 0):
    _need_cuda(codes, c2, c1, mean, W_bf16)
    _check(lib().qlora_nf4_dequant(_ptr(codes), _ptr(c2), _ptr(c1), _ptr(mean), table, N, K, _ptr(W_bf16),
                                   _stream(stream)), "qlora_nf4_dequant")


def qlora_merge(codes, c2, c1, mean, N: int, K: int, A, B, alpha: float, W_out, stream=None, table: int = 0):
    """A [r, K], B [N, r] bf16 device tensors (None for r = 0); W_out bf16 [N, K]."""
    r = 0 if A is None else A.shape[0]
    _need_cuda(codes, c2, c1, mean, A, B, W_out)
    _check(lib().qlora_merge(_ptr(codes), _ptr(c2), _ptr(c1), _ptr(mean), table, N, K, _ptr(A), _ptr(B), r,
                             float(alpha), _ptr(W_out), _stream(stream)), "qlora_merge")


def qlora_linear_fwd_workspace(M: int, N: int, K: int, r: int) -> int:
    return lib().qlora_linear_fwd_workspace(M, N, K, r)


def qlora_linear_fwd(X, codes, c2, c1, mean, A, B, alpha: float, Y, H_out, workspace, N: int,
                     stream=None, table: int = 0):
    _need_cuda(X, codes, c2, c1, mean, A, B, Y, H_out, workspace)
    M, K = X.shape
    r = 0 if A is None else A.shape[0]
    _check(lib().qlora_linear_fwd(_ptr(X), M, N, K, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(mean), table, _ptr(A),
                                  _ptr(B), r, float(alpha), _ptr(Y), _ptr(H_out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "qlora_linear_fwd")


def qlora_linear_fwd_noalloc(X, codes, c2, c1, mean, A, B, alpha: float, Y, H_out, N: int, stream=None,
                             table: int = 0):
    """qlora_linear_fwd with the library's static per-GPU scratch instead of a workspace."""
    _need_cuda(X, codes, c2, c1, mean, A, B, Y, H_out)
    M, K = X.shape
    r = 0 if A is None else A.shape[0]
    _check(lib().qlora_linear_fwd_noalloc(_ptr(X), M, N, K, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(mean), table,
                                          _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(H_out),
                                          _stream(stream)), "qlora_linear_fwd_noalloc")


def qlora_linear_fwd_wait_counter_offset() -> int:
    return lib().qlora_linear_fwd_wait_counter_offset()


def qlora_linear_bwd_workspace(M: int, N: int, K: int, r: int) -> int:
    return lib().qlora_linear_bwd_workspace(M, N, K, r)


def qlora_linear_bwd(dY, X, codes, c2, c1, mean, A, B, alpha: float, H, dX, dA, dB, workspace,
                     stream=None, table: int = 0):
    _need_cuda(dY, X, codes, c2, c1, mean, A, B, H, dX, dA, dB, workspace)
    M, K = X.shape
    N = dY.shape[1]
    r = 0 if A is None else A.shape[0]
    _check(lib().qlora_linear_bwd(_ptr(dY), _ptr(X), M, N, K, _ptr(codes), _ptr(c2), _ptr(c1), _ptr(mean),
                                  table, _ptr(A), _ptr(B), r, float(alpha), _ptr(H), _ptr(dX), _ptr(dA), _ptr(dB),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)), "qlora_linear_bwd")
