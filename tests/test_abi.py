"""Host-side checks of libqlora.so: it loads, exports every entry point that
include/qlora.h declares, and rejects bad arguments before touching a GPU.

No call here reaches a kernel launch: each one fails host validation first
(null or misaligned pointers, bad shapes, small workspaces), so these tests
run on a machine without a GPU.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from bit_nf4_quantized_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libqlora.so not built")

A16 = 0x10000      # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10002      # misaligned fake address


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    names = _declared()
    assert len(names) == 15
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings():
    for s in range(4):
        assert _lib.status_str(s).startswith("QLORA")
    assert "unknown" in _lib.status_str(99)


def test_sizes():
    assert _lib.qlora_nf4_sizes(4096, 4096) == (4096 * 2048, 262144, 1024)
    assert _lib.qlora_nf4_sizes(22016, 8192) == (22016 * 4096, 2818048, 11008)
    assert _lib.qlora_nf4_sizes(1, 64) == (32, 1, 1)
    L = _lib.lib()
    assert L.qlora_nf4_sizes(4, 65, None, None, None) == _lib.QLORA_ESHAPE
    assert L.qlora_nf4_sizes(-1, 64, None, None, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_sizes(0, 0, None, None, None) == _lib.QLORA_OK


def test_library_levels_match_oracle_tables():
    import oracle
    for table, ref in ((0, oracle.nf4_levels_f32()), (1, oracle.uniform4_levels_f32()), (2, oracle.fp4_levels_f32())):
        lv = np.array(_lib.qlora_nf4_levels(table), dtype=np.float32)
        assert np.array_equal(lv.view(np.uint32), np.asarray(ref, np.float32).view(np.uint32)), table
    assert _lib.lib().qlora_nf4_levels(3, None) == _lib.QLORA_EINVAL


def test_quantize_validation():
    L = _lib.lib()
    assert L.qlora_nf4_quantize(None, 4, 64, 0, A16, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize(A16, 4, 64, 0, None, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize(MIS, 4, 64, 0, A16, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize(A16, 4, 64, 0, MIS, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize(A16, 4, 96, 0, A16, A16, None) == _lib.QLORA_ESHAPE
    assert L.qlora_nf4_quantize(A16, -4, 64, 0, A16, A16, None) == _lib.QLORA_EINVAL
    # empty problems are accepted and queue nothing
    assert L.qlora_nf4_quantize(None, 0, 64, 0, None, None, None) == _lib.QLORA_OK
    assert L.qlora_nf4_quantize(None, 8, 0, 0, None, None, None) == _lib.QLORA_OK
    assert L.qlora_nf4_quantize(A16, 4, 64, 3, A16, A16, None) == _lib.QLORA_EINVAL      # unknown table


def test_quantize_bf16_validation():
    L = _lib.lib()
    assert L.qlora_nf4_quantize_bf16(None, 4, 64, 0, A16, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize_bf16(A16, 4, 64, 0, None, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize_bf16(A16 + 4, 4, 64, 0, A16, A16, None) == _lib.QLORA_EINVAL   # W: 8-B aligned
    assert L.qlora_nf4_quantize_bf16(A16, 4, 64, 0, MIS, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize_bf16(A16, 4, 96, 0, A16, A16, None) == _lib.QLORA_ESHAPE
    assert L.qlora_nf4_quantize_bf16(A16, -4, 64, 0, A16, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_quantize_bf16(None, 0, 64, 0, None, None, None) == _lib.QLORA_OK


def test_merge_validation():
    L = _lib.lib()
    f = ctypes.c_float(16.0)
    assert L.qlora_merge(None, A16, A16, A16, 0, 4, 64, A16, A16, 8, f, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_merge(A16, A16, A16, A16, 0, 4, 64, None, A16, 8, f, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_merge(A16, A16, A16, A16, 0, 4, 64, A16, A16, 8, f, MIS, None) == _lib.QLORA_EINVAL
    assert L.qlora_merge(A16, A16, A16, A16, 0, 4, 100, A16, A16, 8, f, A16, None) == _lib.QLORA_ESHAPE
    assert L.qlora_merge(A16, A16, A16, A16, 0, 4, 64, A16, A16, 129, f, A16, None) == _lib.QLORA_ESHAPE
    assert L.qlora_merge(A16, A16, A16, A16, 0, 4, 64, A16, A16, -1, f, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_merge(None, None, None, None, 0, 0, 64, None, None, 8, f, None, None) == _lib.QLORA_OK


def test_double_quant_validation():
    L = _lib.lib()
    need = L.qlora_double_quant_workspace(1000)
    assert need >= 256 * 8
    assert L.qlora_double_quant(A16, 1000, A16, A16, A16, A16, need - 1, None) == _lib.QLORA_EINVAL
    assert L.qlora_double_quant(None, 1000, A16, A16, A16, A16, need, None) == _lib.QLORA_EINVAL
    assert L.qlora_double_quant(A16, 1000, A16, A16, A16, None, need, None) == _lib.QLORA_EINVAL
    assert L.qlora_double_quant(A16 + 2, 1000, A16, A16, A16, A16, need, None) == _lib.QLORA_EINVAL
    assert L.qlora_double_quant(A16, -1, A16, A16, A16, A16, need, None) == _lib.QLORA_EINVAL
    assert L.qlora_double_quant(None, 0, None, None, None, None, 0, None) == _lib.QLORA_OK


def test_dequant_validation():
    L = _lib.lib()
    assert L.qlora_nf4_dequant(None, A16, A16, A16, 0, 4, 64, A16, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_dequant(A16, A16, A16, A16, 0, 4, 64, MIS, None) == _lib.QLORA_EINVAL
    assert L.qlora_nf4_dequant(A16, A16, A16, A16, 0, 4, 100, A16, None) == _lib.QLORA_ESHAPE


def _fwd(L, **kw):
    a = dict(X=A16, M=4, N=64, K=64, codes=A16, c2=A16, c1=A16, mean=A16, A=A16, B=A16, r=8, alpha=16.0,
             Y=A16, H=None, ws=A16, wsb=None, table=0)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = L.qlora_linear_fwd_workspace(max(a["M"], 0), max(a["N"], 0), max(a["K"], 0),
                                                min(max(a["r"], 0), 128))
    return L.qlora_linear_fwd(a["X"], a["M"], a["N"], a["K"], a["codes"], a["c2"], a["c1"], a["mean"],
                              a["table"], a["A"], a["B"], a["r"], a["alpha"], a["Y"], a["H"], a["ws"], a["wsb"],
                              None)


def test_fwd_validation():
    L = _lib.lib()
    assert _fwd(L, K=96) == _lib.QLORA_ESHAPE
    assert _fwd(L, K=0) == _lib.QLORA_ESHAPE
    assert _fwd(L, r=-1) == _lib.QLORA_EINVAL
    assert _fwd(L, r=129) == _lib.QLORA_ESHAPE
    assert _fwd(L, A=None) == _lib.QLORA_EINVAL              # an adapter needs A and B
    assert _fwd(L, B=None) == _lib.QLORA_EINVAL
    # r = 0: no adapter, A and B may be NULL (empty batch: nothing is queued)
    assert _fwd(L, r=0, A=None, B=None, M=0, X=None, Y=None) == _lib.QLORA_OK
    assert _fwd(L, M=-1) == _lib.QLORA_EINVAL
    assert _fwd(L, X=None) == _lib.QLORA_EINVAL
    assert _fwd(L, X=MIS) == _lib.QLORA_EINVAL
    assert _fwd(L, codes=MIS) == _lib.QLORA_EINVAL
    assert _fwd(L, mean=None) == _lib.QLORA_EINVAL
    assert _fwd(L, table=3) == _lib.QLORA_EINVAL
    assert _fwd(L, ws=None) == _lib.QLORA_EINVAL
    assert _fwd(L, ws=A16 + 16) == _lib.QLORA_EINVAL          # workspace must be 256-B aligned
    assert _fwd(L, wsb=1) == _lib.QLORA_EINVAL
    assert _fwd(L, H=A16 + 2) == _lib.QLORA_EINVAL
    assert _fwd(L, M=0, X=None, Y=None) == _lib.QLORA_OK     # empty batch queues nothing
    assert _fwd(L, N=0) == _lib.QLORA_OK
    # M and N beyond 65535 * 128 rows are rejected before any launch
    assert _fwd(L, M=65535 * 128 + 1) == _lib.QLORA_ESHAPE
    assert _fwd(L, N=65535 * 128 + 1) == _lib.QLORA_ESHAPE
    assert L.qlora_linear_fwd_workspace(4, 64, 96, 8) == 0   # invalid shapes report 0
    # decode-sized and large batches both need a workspace
    assert L.qlora_linear_fwd_workspace(1, 4096, 4096, 64) > 256
    assert L.qlora_linear_fwd_workspace(4096, 22016, 8192, 64) >= 4096 * 64 * 4


def test_fwd_noalloc_validation():
    """The no-allocation forward rejects bad arguments and shapes whose
    workspace exceeds its 16 MiB scratch before any device call."""
    L = _lib.lib()
    f = L.qlora_linear_fwd_noalloc
    base = dict(X=A16, M=4, N=64, K=64, codes=A16, c2=A16, c1=A16, mean=A16, table=0, A=A16, B=A16, r=8,
                alpha=16.0, Y=A16, H=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["X"], a["M"], a["N"], a["K"], a["codes"], a["c2"], a["c1"], a["mean"], a["table"], a["A"],
                 a["B"], a["r"], a["alpha"], a["Y"], a["H"], None)

    assert call(K=96) == _lib.QLORA_ESHAPE
    assert call(X=None) == _lib.QLORA_EINVAL
    assert call(X=MIS) == _lib.QLORA_EINVAL
    assert call(table=5) == _lib.QLORA_EINVAL
    assert call(M=0, X=None, Y=None) == _lib.QLORA_OK           # empty batch: nothing queued
    assert L.qlora_linear_fwd_workspace(256, 4096, 4096, 64) > (16 << 20)
    assert call(M=256, N=4096, K=4096, r=64) == _lib.QLORA_ESHAPE


def test_fwd_wait_counter_inside_every_forward_workspace():
    """The wait counter is a 4-byte word at a fixed offset that every forward
    workspace covers (decode-size and tiled shapes alike)."""
    L = _lib.lib()
    off = _lib.qlora_linear_fwd_wait_counter_offset()
    assert off % 4 == 0
    for shape in ((1, 64, 64, 0), (1, 4096, 4096, 64), (16, 11008, 4096, 64), (17, 64, 64, 1),
                  (4096, 22016, 8192, 64)):
        assert L.qlora_linear_fwd_workspace(*shape) >= off + 4, shape


def test_bwd_validation():
    L = _lib.lib()
    need = L.qlora_linear_bwd_workspace(32, 64, 128, 8)
    assert need >= 2 * 32 * 8 * 4

    def call(**kw):
        a = dict(dY=A16, X=A16, M=32, N=64, K=128, codes=A16, c2=A16, c1=A16, mean=A16, A=A16, B=A16, r=8,
                 alpha=16.0, H=None, dX=A16, dA=A16, dB=A16, ws=A16, wsb=need, table=0)
        a.update(kw)
        return L.qlora_linear_bwd(a["dY"], a["X"], a["M"], a["N"], a["K"], a["codes"], a["c2"], a["c1"],
                                  a["mean"], a["table"], a["A"], a["B"], a["r"], a["alpha"], a["H"], a["dX"],
                                  a["dA"], a["dB"], a["ws"], a["wsb"], None)

    assert call(K=100) == _lib.QLORA_ESHAPE
    assert call(r=200) == _lib.QLORA_ESHAPE
    assert call(dY=None) == _lib.QLORA_EINVAL
    assert call(dA=None) == _lib.QLORA_EINVAL
    assert call(dB=None) == _lib.QLORA_EINVAL
    assert call(dX=MIS) == _lib.QLORA_EINVAL
    assert call(wsb=need - 1) == _lib.QLORA_EINVAL
    assert call(A=None) == _lib.QLORA_EINVAL
    assert call(table=3) == _lib.QLORA_EINVAL
    assert call(table=-1) == _lib.QLORA_EINVAL
    # no adapter and an empty batch: nothing to compute, nothing queued
    assert call(r=0, A=None, B=None, dA=None, dB=None, M=0, dY=None, X=None) == _lib.QLORA_OK


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.lib()


def test_save_load_quantized_round_trip(tmp_path):
    """The quantized tensor is the artifact: it round-trips through .npz bit
    for bit (host tensors here; the device copies are plain transfers), and a
    file of the wrong shape is refused."""
    import torch
    import bit_nf4_quantized_quant_amd as qa
    N, K = 5, 192
    rng = np.random.default_rng(3)
    code_bytes, n_c2, n_c1 = _lib.qlora_nf4_sizes(N, K)
    q = qa.QuantizedWeight(N, K, torch.from_numpy(rng.integers(0, 256, (N, K // 2), dtype=np.uint8)),
                           torch.from_numpy(rng.random(n_c2, dtype=np.float32)),
                           torch.from_numpy(rng.integers(0, 256, n_c2, dtype=np.uint8)),
                           torch.from_numpy(rng.random(n_c1, dtype=np.float32)),
                           torch.tensor([0.125], dtype=torch.float32), 2)
    path = str(tmp_path / "w.npz")
    qa.save_quantized(q, path)
    r = qa.load_quantized(path, device="cpu")
    assert (r.N, r.K, r.table) == (N, K, 2)
    for a, b in ((q.codes, r.codes), (q.absmax, r.absmax), (q.c2, r.c2), (q.c1, r.c1), (q.mean, r.mean)):
        assert a.dtype == b.dtype and torch.equal(a, b)
    bad = str(tmp_path / "bad.npz")
    np.savez(bad, N=np.int64(N), K=np.int64(K + 64), table=np.int64(0), codes=q.codes.numpy(), c2=q.c2.numpy(),
             c1=q.c1.numpy(), mean=q.mean.numpy())
    with pytest.raises(ValueError):
        qa.load_quantized(bad, device="cpu")


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; asked for more it says so and exits with 2."""
    import json
    import subprocess
    import sys
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert run.returncode == 2
    msg = json.loads(run.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
