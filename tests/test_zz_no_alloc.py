"""The no-allocation forward (qlora_linear_fwd_noalloc) through the C ABI
against the workspace forward (qlora_linear_fwd) on the same inputs: two
calls in a row, the second with a smaller input, on the decode path
(M <= 16: the matrix-core kernel, then the GEMV) and on the tiled path; the
outputs must equal the workspace forward's bit for bit (both run the same
kernels, whose sums have a fixed order) and meet the layer's tolerance
against the oracle.  A shape whose workspace exceeds the scratch is
rejected before any launch."""

import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_f64, check_close, dev_bf16, dev_f32, host, host_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - the GPU suite needs an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import bit_nf4_quantized_quant_amd as qa  # noqa: E402
from bit_nf4_quantized_quant_amd import _lib  # noqa: E402

L = qa.lib()
L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
L.qlora_linear_fwd_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]


def p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc_fwd(X, q, A, B, alpha, Y, H):
    M, K = X.shape
    r = 0 if A is None else A.shape[0]
    return L.qlora_linear_fwd_noalloc(p(X), M, q.N, K, p(q.codes), p(q.c2), p(q.c1), p(q.mean), q.table, p(A),
                                      p(B), r, alpha, p(Y), p(H),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def layer(M, N, K, r, seed):
    d = synth.make_layer(synth.LayerShape("t", M=M, N=N, K=K, r=r, seed_offset=seed))
    q = qa.quantize(dev_f32(d["W"]))
    ref = oracle.quantize_layer(d["W"])
    wd = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K)
    return d, q, wd


@pytest.mark.parametrize("first,second", [((16, 4096, 4096, 64), (1, 1024, 1024, 16)),
                                          ((64, 2048, 1024, 16), (40, 512, 512, 8))])
def test_noalloc_forward_matches_workspace_forward(first, second):
    for i, (M, N, K, r) in enumerate((first, second)):
        print(f"[noalloc] call {i}: M={M} N={N} K={K} r={r}", flush=True)
        d, q, wd = layer(M, N, K, r, 6100 + 10 * i + M)
        X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        H = torch.empty((M, r), dtype=torch.float32, device="cuda")
        st = noalloc_fwd(X, q, A, B, 16.0, Y, H)
        assert st == 0, _lib.status_str(st)
        Yw, Hw = qa.linear_fwd(X, q, A, B, 16.0)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Yw.view(torch.int16)), "Y differs from the workspace forward"
        assert torch.equal(H, Hw), "H differs from the workspace forward"
        Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], 16.0, r)
        check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y")
        check_close(host(H), Hr, "H")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    M, N, K, r = 256, 4096, 4096, 64
    assert L.qlora_linear_fwd_workspace(M, N, K, r) > (16 << 20)
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = L.qlora_linear_fwd_noalloc(p(dummy), M, N, K, p(dummy), p(dummy), p(dummy), p(dummy), 0, p(dummy),
                                    p(dummy), r, 16.0, p(dummy), None, None)
    assert st == _lib.QLORA_ESHAPE
