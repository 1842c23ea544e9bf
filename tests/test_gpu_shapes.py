"""GPU parity over a seeded sweep of layer shapes: the forward and backward
against the CPU oracle on 48 shapes drawn once from a fixed seed, so that the
launchers' choices (GEMV with 16- or 32-row tiles, the matrix-core decode
kernel and its K slices, 128 x 128 tiles with split-K, the single pass over
dY for dH and dB or the separate products, element-wise or 16-byte loads)
meet ragged sizes in combinations the hand-picked cases do not; and a second
seeded sweep of 16 decode-size forwards (M <= 16) that also checks that no
bounded cross-workgroup wait gave up.  Same tolerances as the other parity
tests."""

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

qa.lib()


def _shapes(n=48, seed=20261203):
    rng = np.random.default_rng(seed)
    ms = [1, 2, 3, 4, 5, 8, 12, 16, 17, 24, 40, 64, 100, 128, 200, 256, 300, 513, 600]
    rs = [1, 5, 8, 16, 24, 32, 40, 56, 64, 72, 96, 128]
    out = []
    for i in range(n):
        M = int(rng.choice(ms))
        # N: a multiple of 8 two times in three (the single pass needs it), else ragged
        N = int(rng.integers(1, 88)) * 8 if rng.random() < 2 / 3 else int(rng.integers(1, 700))
        K = 64 * int(rng.integers(1, 25))
        r = int(rng.choice(rs))
        out.append((M, N, K, r, i))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("M,N,K,r,i", SHAPES)
def test_forward_backward_shape_sweep(M, N, K, r, i):
    print(f"[sweep {i}] M={M} N={N} K={K} r={r}", flush=True)
    alpha = 16.0
    d = synth.make_layer(synth.LayerShape("sweep", M=M, N=N, K=K, r=r, seed_offset=50000 + i), with_dy=True)
    ref = oracle.quantize_layer(d["W"])
    wd = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K)
    q = qa.quantize(dev_f32(d["W"]))
    X, A, B, dY = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"]), dev_bf16(d["dY"])
    Y, H = qa.linear_fwd(X, q, A, B, alpha)
    dX, dA, dB = qa.linear_bwd(dY, X, q, A, B, alpha, H=H if i % 2 == 0 else None)
    torch.cuda.synchronize()
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y")
    check_close(host(H), Hr, "H")
    g = oracle.linear_bwd(d["dY"], d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(dX)), g["dX"], "dX")
    check_close(bf16_f64(host_bf16_bits(dA)), g["dA"], "dA", bf16_floor=True if M == 1 else "auto")
    check_close(bf16_f64(host_bf16_bits(dB)), g["dB"], "dB", bf16_floor=True if M == 1 else "auto")


def _decode_shapes(n=16, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 17))
        N = int(rng.integers(8, 1025)) * 8 if rng.random() < 3 / 4 else int(rng.integers(1, 8192))
        K = 64 * int(rng.integers(1, 65))
        r = int(rng.choice([1, 4, 8, 16, 32, 40, 64, 96, 128]))
        out.append((M, N, K, r, i))
    return out


DECODE_SHAPES = _decode_shapes()


@pytest.mark.parametrize("M,N,K,r,i", DECODE_SHAPES)
def test_decode_forward_shape_sweep(M, N, K, r, i):
    """Decode-size forwards (M <= 16: the GEMV with 16- or 32-row tiles, the
    matrix-core decode kernel and its K slices) on 16 seeded shapes up to
    8192 x 4096, every output of Y and H against the oracle, and no bounded
    wait for a partial result may give up."""
    print(f"[decode sweep {i}] M={M} N={N} K={K} r={r}", flush=True)
    alpha = 16.0
    d = synth.make_layer(synth.LayerShape("dsweep", M=M, N=N, K=K, r=r, seed_offset=60000 + i))
    ref = oracle.quantize_layer(d["W"])
    wd = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K)
    q = qa.quantize(dev_f32(d["W"]))
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    ws = qa.fwd_workspace(M, N, K, r, "cuda")
    before = qa.fwd_wait_count(ws)
    Y, H = qa.linear_fwd(X, q, A, B, alpha, workspace=ws)
    torch.cuda.synchronize()
    assert qa.fwd_wait_count(ws) == before, "a wait for a partial result gave up"
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y")
    check_close(host(H), Hr, "H")
