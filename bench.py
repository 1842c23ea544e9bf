"""Benchmark of the QLoRA NF4 linear on one MI355X.

Headline (the `value` of the JSON line): forward HBM throughput at M = 1 on
the 4096 x 4096 decode layer (NF4 weight + double-quantized constants, LoRA
r = 64, alpha = 16), with inputs resident in HBM and the weights rotated over
enough distinct copies (> 512 MB) that every call streams its weight from HBM
rather than from the 256 MB Infinity Cache.  A step is one forward call of the
layer (one kernel launch); the timed steps are captured in a HIP graph and
replayed once between HIP events, so host launch cost stays out of the figure.

Also measured in the same run and reported under "extra": M = 4 and 16 on the
decode layer, the Llama-7B MLP shapes at M = 1, 16 and 256, the 65B-scale
training layer (22016 x 8192, M = 4096) forward and backward in TFLOP/s,
quantize + double quant throughput, and the 7B-shaped decoder's 224 linears
(quantize all, then one forward pass at M = 1 and at M = 512).  The CPU oracle is timed on a bounded sample of the
headline workload (`cpu_baseline`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--eager] [--no-cpu]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd: HBM GB/s at M=1, TFLOP/s at M=4096 (% of peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, public spec
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, public spec
MALL_BYTES = 256 << 20
FP64_PEAK_TFLOPS = 78.6   # MI355X fp64 vector peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic work

def weight_bytes(N, K):
    """Packed codes + c2 + c1 + mean of one quantized weight."""
    n_c2 = N * K // 64
    return N * K // 2 + n_c2 + 4 * ((n_c2 + 255) // 256) + 4


def fwd_bytes(M, N, K, r):
    """Algorithmic HBM bytes of one forward: W once, X, Y, A, B in bf16 once each."""
    return weight_bytes(N, K) + 2 * M * K + 2 * M * N + 2 * r * K + 2 * N * r


def fwd_flops(M, N, K, r):
    return 2 * M * N * K + 2 * M * r * (K + N)


def bwd_flops(M, N, K, r):
    # dX main + H recompute-free: dH (2MNr), dB (2MNr), dA (2MrK), dX LoRA (2MrK), dX main (2MNK)
    return 2 * M * N * K + 4 * M * N * r + 4 * M * r * K


def bwd_bytes(M, N, K, r):
    return weight_bytes(N, K) + 2 * M * N + 2 * M * K * 2 + 4 * M * r + 2 * r * K * 2 + 2 * N * r * 2


# ----------------------------------------------------------------------------- GPU helpers

def make_layer_gpu(torch, qa, N, K, r, copies, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    W = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
    q = qa.quantize(W)
    del W
    A = (torch.randn((r, K), generator=gen, device="cuda") / K).to(torch.bfloat16)
    B = (torch.randn((N, r), generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    sets = []
    for i in range(copies):
        qi = qa.QuantizedWeight(N, K, q.codes.clone(), q.absmax, q.c2.clone(), q.c1.clone(), q.mean.clone())
        sets.append((qi, A.clone(), B.clone()))
    torch.cuda.synchronize()
    return sets


def timed_graph(torch, fn, steps, warmup):
    """Run fn(i) warmup times eagerly, capture `steps` calls in one graph, replay it
    between events; returns ms per call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(warmup):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    torch.cuda.synchronize()
    g.replay()                      # one untimed replay
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def timed_eager(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def calib_lib():
    """The reference kernels of libqlora_calib.so (empty kernel, plain read)."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "bit_nf4_quantized_quant_amd", "libqlora_calib.so"))
    L.calib_empty.restype = ctypes.c_int
    L.calib_empty.argtypes = [ctypes.c_void_p]
    L.calib_read.restype = ctypes.c_int
    L.calib_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return L


def bench_attainable(torch, nbytes, copies, steps, warmup):
    """What the platform allows in the headline's own timing mode (HIP graph
    replay): an empty kernel's launch-to-launch time, and a plain streaming
    read of the same byte count rotated over the same number of copies (best
    over a few workgroup counts), plus the read bandwidth of a 1 GiB buffer."""
    import ctypes
    L = calib_lib()

    def cur():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"calibration kernel launch failed: hipError {rc}")

    ms_empty = timed_graph(torch, lambda i: ok(L.calib_empty(cur())), steps, warmup)
    n16 = (nbytes + 15) // 16 * 16
    bufs = [torch.empty(n16, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = None
    for wgs in (256, 512, 1024, 2048):
        ms = timed_graph(torch, lambda i: ok(L.calib_read(bufs[i % copies].data_ptr(), n16, wgs,
                                                          sink.data_ptr(), cur())), steps, warmup)
        if best is None or ms < best[0]:
            best = (ms, wgs)
    del bufs
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    ms_big = timed_graph(torch, lambda i: ok(L.calib_read(big.data_ptr(), big.numel(), 8192, sink.data_ptr(),
                                                          cur())), 10, 2)
    del big
    return {"mode": "graph replay, same as the headline",
            "empty_kernel_us": ms_empty * 1e3,
            "stream_same_bytes_us": best[0] * 1e3, "stream_same_bytes_GBps": n16 / best[0] / 1e6,
            "stream_same_bytes_workgroups": best[1], "stream_same_bytes_copies": copies,
            "stream_1GiB_GBps": (1 << 30) / ms_big / 1e6}


def bench_fwd(torch, qa, M, N, K, r, steps, warmup, copies, seed=0, graph=True):
    sets = make_layer_gpu(torch, qa, N, K, r, copies, seed)
    xs = [torch.randn((M, K), device="cuda").to(torch.bfloat16) for _ in range(copies)]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    H = torch.empty((M, r), dtype=torch.float32, device="cuda")
    ws = qa.fwd_workspace(M, N, K, r, "cuda")

    def call(i):
        q, A, B = sets[i % copies]
        qa.qlora_linear_fwd(xs[i % copies], q.codes, q.c2, q.c1, q.mean, A, B, 16.0, Y, H, ws, N)

    ms = (timed_graph if graph else timed_eager)(torch, call, steps, warmup)
    # no decode launch fell back to computing H itself (that would be the slow path)
    giveups = qa.fwd_wait_count(ws)
    if giveups:
        raise RuntimeError(f"M={M} {N}x{K}: {giveups} waits for partial results gave up (slow fallback ran)")
    byts = fwd_bytes(M, N, K, r)
    fl = fwd_flops(M, N, K, r)
    del sets, xs
    return {"M": M, "N": N, "K": K, "r": r, "ms": ms, "GBps": byts / ms / 1e6, "TFLOPs": fl / ms / 1e9,
            "hbm_frac": byts / ms / 1e6 / HBM_PEAK_GBS, "mfma_frac": fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS,
            "bytes": byts, "flops": fl, "copies": copies}


def bench_bwd(torch, qa, M, N, K, r, steps, warmup, seed=0):
    sets = make_layer_gpu(torch, qa, N, K, r, 1, seed)
    q, A, B = sets[0]
    X = torch.randn((M, K), device="cuda").to(torch.bfloat16)
    dY = torch.randn((M, N), device="cuda").to(torch.bfloat16)
    H = torch.empty((M, r), dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws_f = qa.fwd_workspace(M, N, K, r, "cuda")
    qa.qlora_linear_fwd(X, q.codes, q.c2, q.c1, q.mean, A, B, 16.0, Y, H, ws_f, N)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((N, r), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(qa.qlora_linear_bwd_workspace(M, N, K, r), dtype=torch.uint8, device="cuda")

    def call(i):
        qa.qlora_linear_bwd(dY, X, q.codes, q.c2, q.c1, q.mean, A, B, 16.0, H, dX, dA, dB, ws)

    ms = timed_eager(torch, call, steps, warmup)
    fl = bwd_flops(M, N, K, r)
    return {"M": M, "N": N, "K": K, "r": r, "ms": ms, "TFLOPs": fl / ms / 1e9,
            "mfma_frac": fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, "flops": fl}


def bench_quantize(torch, qa, N, K, steps, warmup):
    W = torch.randn((N, K), device="cuda", dtype=torch.float32) * 0.02
    code_bytes, n_c2, n_c1 = qa.qlora_nf4_sizes(N, K)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    absmax = torch.empty(n_c2, dtype=torch.float32, device="cuda")
    c2 = torch.empty(n_c2, dtype=torch.uint8, device="cuda")
    c1 = torch.empty(n_c1, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(qa.qlora_double_quant_workspace(n_c2), dtype=torch.uint8, device="cuda")
    ms_q = timed_eager(torch, lambda i: qa.qlora_nf4_quantize(W, codes, absmax), steps, warmup)
    Wb = W.to(torch.bfloat16)
    ms_qb = timed_eager(torch, lambda i: qa.qlora_nf4_quantize_bf16(Wb, codes, absmax), steps, warmup)
    ms_dq = timed_eager(torch, lambda i: qa.qlora_double_quant(absmax, c2, c1, mean, ws), steps, warmup)
    qbytes = N * K * 4 + N * K // 2 + 4 * n_c2
    qbytes_b = N * K * 2 + N * K // 2 + 4 * n_c2
    return {"N": N, "K": K, "quantize_ms": ms_q, "quantize_GBps": qbytes / ms_q / 1e6,
            "quantize_hbm_frac": qbytes / ms_q / 1e6 / HBM_PEAK_GBS,
            "quantize_bf16_ms": ms_qb, "quantize_bf16_GBps": qbytes_b / ms_qb / 1e6,
            "quantize_bf16_hbm_frac": qbytes_b / ms_qb / 1e6 / HBM_PEAK_GBS, "double_quant_ms": ms_dq,
            "double_quant_GBps": (5 * n_c2 + 4 * n_c1) / ms_dq / 1e6}


def bench_merge(torch, qa, N, K, r, steps, warmup):
    """Merge W_deq + s B A into a bf16 weight: fp64 multiply-adds, r per weight."""
    sets = make_layer_gpu(torch, qa, N, K, r, 1, 7)
    q, A, B = sets[0]
    out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    ms = timed_eager(torch, lambda i: qa.qlora_merge(q.codes, q.c2, q.c1, q.mean, N, K, A, B, 16.0, out),
                     steps, warmup)
    fl = 2 * N * K * r
    return {"N": N, "K": K, "r": r, "ms": ms, "fp64_TFLOPs": fl / ms / 1e9,
            "fp64_frac": fl / ms / 1e9 / FP64_PEAK_TFLOPS, "GBps": (N * K * 2.5 + N * K / 64) / ms / 1e6}


def bench_decoder(torch, qa, reps, seed=5):
    """The 7B-shaped decoder's linears (32 layers x q, k, v, o, gate, up, down;
    LoRA r = 16 on q and v): quantize + double quant all of them, then one
    forward pass over all 224 linears at M = 1 and at M = 512."""
    import synth
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    layers = []
    ms_quant = 0.0
    params = 0
    for _ in range(synth.DECODER_LAYERS):
        for mod, N, K, r in synth.DECODER_MODULES:
            W = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            q = qa.quantize(W)
            e1.record()
            torch.cuda.synchronize()
            ms_quant += e0.elapsed_time(e1)
            params += N * K
            del W
            A = B = None
            if r:
                A = (torch.randn((r, K), generator=gen, device="cuda") / K).to(torch.bfloat16)
                B = (torch.randn((N, r), generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
            layers.append((q, A, B, N, K, r))
    log(f"[bench] decoder: {len(layers)} linears quantized, {ms_quant:.1f} ms")
    res = {"params": params, "quantize_ms": ms_quant,
           "quantize_GBps": params * (4 + 0.5 + 4 / 64) / ms_quant / 1e6}
    for M in (1, 512):
        xs = {K: torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16) for K in (4096, 11008)}
        ys = {N: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for N in (4096, 11008)}
        ws = qa.fwd_workspace(M, 11008, 11008, 16, "cuda")

        def one_pass(i):
            for q, A, B, N, K, r in layers:
                qa.qlora_linear_fwd(xs[K], q.codes, q.c2, q.c1, q.mean, A, B, 16.0, ys[N], None, ws, N)

        ms = (timed_graph if M == 1 else timed_eager)(torch, one_pass, reps, 1)
        byts = sum(fwd_bytes(M, N, K, r) for _, _, _, N, K, r in layers)
        fl = sum(fwd_flops(M, N, K, r) for _, _, _, N, K, r in layers)
        res[f"m{M}"] = {"ms": ms, "GBps": byts / ms / 1e6, "TFLOPs": fl / ms / 1e9,
                        "hbm_frac": byts / ms / 1e6 / HBM_PEAK_GBS,
                        "mfma_frac": fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, "bytes": byts, "flops": fl}
        log(f"[bench] decoder pass M={M}: {ms:.3f} ms")
        del xs, ys, ws
    del layers
    res["fused"] = bench_decoder_fused(torch, qa, reps, gen)
    return res


def bench_decoder_fused(torch, qa, reps, gen):
    """The same decoder with q|k|v and gate|up concatenated along N (128
    launches per pass instead of 224; the q and v adapters as one rank-32
    adapter with block-structured B), one pass at M = 1 and M = 512."""
    import synth
    layers = []
    for _ in range(synth.DECODER_LAYERS):
        for mod, N, K, r in synth.DECODER_FUSED:
            W = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
            q = qa.quantize(W)
            del W
            A = B = None
            if r:
                A = (torch.randn((r, K), generator=gen, device="cuda") / K).to(torch.bfloat16)
                B = (torch.randn((N, r), generator=gen, device="cuda") * 0.01)
                B = (B * torch.from_numpy(synth.fused_qkv_b_mask(N, r)).to("cuda")).to(torch.bfloat16)
            layers.append((q, A, B, N, K, r))
    res = {"launches_per_pass": len(layers)}
    for M in (1, 512):
        xs = {K: torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16) for K in (4096, 11008)}
        ys = {N: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for N in (4096, 12288, 22016)}
        need = max(qa.qlora_linear_fwd_workspace(M, N, K, r) for _, N, K, r in synth.DECODER_FUSED)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")

        def one_pass(i):
            for q, A, B, N, K, r in layers:
                qa.qlora_linear_fwd(xs[K], q.codes, q.c2, q.c1, q.mean, A, B,
                                    synth.FUSED_QKV_ALPHA if r else 16.0, ys[N], None, ws, N)

        ms = (timed_graph if M == 1 else timed_eager)(torch, one_pass, reps, 1)
        byts = sum(fwd_bytes(M, N, K, r) for _, _, _, N, K, r in layers)
        fl = sum(fwd_flops(M, N, K, r) for _, _, _, N, K, r in layers)
        res[f"m{M}"] = {"ms": ms, "GBps": byts / ms / 1e6, "TFLOPs": fl / ms / 1e9,
                        "hbm_frac": byts / ms / 1e6 / HBM_PEAK_GBS,
                        "mfma_frac": fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS}
        log(f"[bench] fused decoder pass M={M}: {ms:.3f} ms")
        del xs, ys, ws
    del layers
    return res


# ----------------------------------------------------------------------------- traffic from counters

def plain_gemm_reference(torch, M, N, K, steps=5):
    """The stack's own dense bf16 GEMM (torch.matmul, dispatched to hipBLASLt) on
    the same M x N x K, timed with HIP events, with the weight stored [K][N] and
    [N][K] (the layer's own layout, multiplied as its transpose); the faster
    is the reference for what the matrix cores reach on this shape without
    any dequantization.  It is not part of the layer's path."""
    x = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
    out = {"what": "torch.matmul bf16 (hipBLASLt), same M x N x K, no dequantization"}
    for name, w, op in (("w_kn", torch.randn(K, N, device="cuda", dtype=torch.bfloat16), lambda w: w),
                        ("w_nk", torch.randn(N, K, device="cuda", dtype=torch.bfloat16), lambda w: w.t())):
        for _ in range(2):
            torch.matmul(x, op(w))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.matmul(x, op(w))
        e1.record()
        torch.cuda.synchronize()
        out[f"{name}_ms"] = e0.elapsed_time(e1) / steps
        del w
    del x
    out["ms"] = min(out["w_kn_ms"], out["w_nk_ms"])
    out["TFLOPs"] = 2.0 * M * N * K / (out["ms"] * 1e-3) / 1e12
    return out


def plain_dx_reference(torch, M, N, K, steps=5):
    """The stack's dense bf16 GEMM on the backward's dX shape, dY [M,N] times the
    weight [N,K] as stored (torch.matmul, hipBLASLt), timed with HIP events: a
    reference for the dX product, which takes most of the backward.  It is not
    part of the layer's path."""
    dy = torch.randn(M, N, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
    for _ in range(2):
        torch.matmul(dy, w)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.matmul(dy, w)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del dy, w
    return {"what": "torch.matmul bf16 (hipBLASLt) of dY [M,N] and W [N,K], no dequantization", "ms": ms,
            "TFLOPs": 2.0 * M * N * K / (ms * 1e-3) / 1e12}


def kernel_source_hash(names):
    """sha256[:16] over the kernel's source files, concatenated in order."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "bit_nf4_quantized_quant_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(summary_name, source_names):
    """HBM bytes per launch recorded in a profiles/ summary, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source sha256\[:16\]:\s*([0-9a-f]+)", text)
    m_traf = re.search(r"HBM traffic per launch \(bytes\):\s*([0-9.e+]+)", text)
    if not m_hash or not m_traf or m_hash.group(1) != kernel_source_hash(source_names):
        return None
    return float(m_traf.group(1))


# ----------------------------------------------------------------------------- CPU oracle

def cpu_description():
    """CPU model, cores available to this process, and the BLAS pools numpy uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)), "blas_pools": blas}


def cpu_baseline(budget_s=12.0, side_budget_s=4.0):
    """The oracle, single-threaded, on bounded samples: the headline forward
    (rows of the 4096x4096 decode layer at M = 1) gives `value`; quantize +
    double quant on a row slice of the same layer and the backward on a slice
    of the 65B-scale layer (256 rows of X and dY, 256 rows of W) are reported
    beside it."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle
    import synth

    shape = synth.DECODE[0]
    d = synth.make_layer(shape)
    q = oracle.quantize_layer(d["W"])
    rows_per = 256
    rng = np.random.default_rng(0)
    done_rows = 0
    t_total = 0.0
    desc = cpu_description()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        while t_total < budget_s:
            rows = np.sort(rng.choice(shape.N, rows_per, replace=False))
            t0 = time.perf_counter()
            wd = oracle.dequant_weight(q["codes"], q["c2"], q["c1"], q["mu"], shape.N, shape.K, rows=rows)
            oracle.linear_fwd(d["X"], wd, d["A"], d["B"][rows], shape.alpha, shape.r)
            t_total += time.perf_counter() - t0
            done_rows += rows_per
        # quantize + double quant of 256-row slices of the same weight
        t_q, q_rows = 0.0, 0
        while t_q < side_budget_s:
            r0 = (q_rows // rows_per) * rows_per % shape.N
            t0 = time.perf_counter()
            oracle.quantize_layer(d["W"][r0:r0 + rows_per])
            t_q += time.perf_counter() - t0
            q_rows += rows_per
        q_params = q_rows * shape.K
        q_bytes = q_params * 4 + q_params // 2 + 4 * (q_params // 64)
        # backward on a slice of the 65B-scale layer: 256 rows of X/dY, 256 rows of W
        tr = synth.TRAIN65B
        Ms, Ns = 256, 256
        Xs = synth.f32_to_bf16_bits(synth.normal_f32(7001, (Ms, tr.K), 1.0))
        dYs = synth.f32_to_bf16_bits(synth.normal_f32(7002, (Ms, Ns), 1.0))
        Ws = synth.normal_f32(7003, (Ns, tr.K), 0.02)
        As = synth.f32_to_bf16_bits(synth.normal_f32(7004, (tr.r, tr.K), 1.0 / tr.K))
        Bs = synth.f32_to_bf16_bits(synth.normal_f32(7005, (Ns, tr.r), 0.01))
        qs = oracle.quantize_layer(Ws)
        wds = oracle.dequant_weight(qs["codes"], qs["c2"], qs["c1"], qs["mu"], Ns, tr.K)
        t_b, n_b = 0.0, 0
        while t_b < side_budget_s:
            t0 = time.perf_counter()
            oracle.linear_bwd(dYs, Xs, wds, As, Bs, tr.alpha, tr.r)
            t_b += time.perf_counter() - t0
            n_b += 1
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    frac = done_rows / shape.N
    byts = fwd_bytes(shape.M, shape.N, shape.K, shape.r) * frac
    res = {"value": byts / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{done_rows} output rows (in blocks of {rows_per}) of decode_4096x4096_m1, "
                     f"oracle dequant + fp64 forward, {t_total:.1f} s single-threaded; bytes scaled "
                     f"by the row fraction",
           "quantize_dq": {"GBps": q_bytes / t_q / 1e9, "params": q_params, "s": t_q,
                           "sample": f"quantize + double quant of {rows_per}-row slices of the 4096x4096 weight"},
           "backward": {"GFLOPs": n_b * bwd_flops(Ms, Ns, tr.K, tr.r) / t_b / 1e9, "calls": n_b, "s": t_b,
                        "sample": f"dX, dA, dB of the 65B-scale layer's shape restricted to M={Ms} rows of X/dY "
                                  f"and N={Ns} rows of W (K={tr.K}, r={tr.r}), fp64"}}
    res.update(desc)
    res["blas_threads_used"] = 1 if threadpool_limits else None
    return res


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the empty-kernel and plain-read reference timings")
    ap.add_argument("--eager", action="store_true",
                    help="launch the headline steps one by one instead of replaying a graph "
                         "(for per-dispatch counter collection)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--train65b-only", action="store_true",
                    help="only the 65B-scale layer's forward and backward, --steps calls each, no JSON line "
                         "(for matrix-core counter runs)")
    ap.add_argument("--decode-sizes-only", action="store_true",
                    help="only the 4096x4096 forward at (M, r) = (1, 64), (8, 0), (8, 64), (16, 0), (16, 64), "
                         "launched one by one, 2 warmup and --steps calls each, no JSON line "
                         "(for per-dispatch counter runs of the decode kernels)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import bit_nf4_quantized_quant_amd as qa
    qa.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), CUs {props.multi_processor_count}")

    if args.train65b_only:
        import synth
        sh = synth.TRAIN65B
        f = bench_fwd(torch, qa, sh.M, sh.N, sh.K, sh.r, args.steps, 1, 1, graph=False)
        b = bench_bwd(torch, qa, sh.M, sh.N, sh.K, sh.r, args.steps, 1)
        log(f"[bench] {sh.name}: fwd {f['ms']:.3f} ms ({f['TFLOPs']:.0f} TFLOP/s), "
            f"bwd {b['ms']:.3f} ms ({b['TFLOPs']:.0f} TFLOP/s)")
        return

    if args.decode_sizes_only:
        for M, rr in ((1, 64), (8, 0), (8, 64), (16, 0), (16, 64)):
            cp = max(2, int(2 * MALL_BYTES / fwd_bytes(M, 4096, 4096, rr)) + 1)
            res = bench_fwd(torch, qa, M, 4096, 4096, rr, args.steps, 2, cp, graph=False)
            log(f"[bench] 4096x4096 M={M} r={rr}: {res['ms'] * 1e3:.2f} us/call")
        return

    N, K, r = 4096, 4096, 64
    copies = max(2, int(2 * MALL_BYTES / fwd_bytes(1, N, K, r)) + 1)
    log(f"[bench] decode fwd M=1 {N}x{K} r={r}: {copies} weight copies, {args.steps} steps")
    head = bench_fwd(torch, qa, 1, N, K, r, args.steps, args.warmup, copies, graph=not args.eager)
    log(f"[bench] M=1: {head['ms'] * 1e3:.2f} us/call, {head['GBps']:.0f} GB/s")

    if args.copy_calibration:
        a = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    extra = {}
    plain = None
    if not args.quick:
        for M in (4, 16):
            res = bench_fwd(torch, qa, M, N, K, r, args.steps, args.warmup, copies)
            extra[f"decode_4096x4096_m{M}"] = res
            log(f"[bench] M={M}: {res['ms'] * 1e3:.2f} us/call, {res['GBps']:.0f} GB/s")
        for nm, n, k in (("mlp_gate_up_11008x4096", 11008, 4096), ("mlp_down_4096x11008", 4096, 11008)):
            for M in (1, 16, 256):
                cp = max(2, int(2 * MALL_BYTES / fwd_bytes(M, n, k, r)) + 1)
                res = bench_fwd(torch, qa, M, n, k, r, args.steps, args.warmup, cp)
                extra[f"{nm}_m{M}"] = res
                log(f"[bench] {nm} M={M}: {res['ms'] * 1e3:.2f} us/call, {res['GBps']:.0f} GB/s, "
                    f"{res['TFLOPs']:.1f} TFLOP/s")
        Ml, Nl, Kl = 4096, 22016, 8192
        res = bench_fwd(torch, qa, Ml, Nl, Kl, r, 10, 2, 3, graph=False)
        extra["train65b_22016x8192_m4096_fwd"] = res
        log(f"[bench] 65B layer fwd M=4096: {res['ms']:.3f} ms, {res['TFLOPs']:.0f} TFLOP/s")
        plain = plain_gemm_reference(torch, Ml, Nl, Kl)
        log(f"[bench] plain bf16 GEMM {Ml}x{Nl}x{Kl}: {plain['ms']:.3f} ms, {plain['TFLOPs']:.0f} TFLOP/s")
        res = bench_bwd(torch, qa, Ml, Nl, Kl, r, 5, 1)
        res["plain_dx_gemm"] = plain_dx_reference(torch, Ml, Nl, Kl)
        extra["train65b_22016x8192_m4096_bwd"] = res
        log(f"[bench] 65B layer bwd M=4096: {res['ms']:.3f} ms, {res['TFLOPs']:.0f} TFLOP/s")
        res = bench_quantize(torch, qa, Nl, Kl, 5, 1)
        extra["quantize_22016x8192"] = res
        log(f"[bench] quantize: {res['quantize_GBps']:.0f} GB/s (bf16 input {res['quantize_bf16_GBps']:.0f} GB/s), "
            f"double quant {res['double_quant_ms'] * 1e3:.1f} us")
        res = bench_merge(torch, qa, 4096, 4096, 64, 20, 3)
        extra["merge_4096x4096_r64"] = res
        log(f"[bench] merge 4096x4096 r=64: {res['ms'] * 1e3:.1f} us, {res['fp64_TFLOPs']:.1f} fp64 TFLOP/s")
        torch.cuda.empty_cache()
        res = bench_decoder(torch, qa, 20)
        extra["decoder_7b_224_linears"] = res
        log(f"[bench] 7B decoder: quantize {res['params'] / 1e9:.2f}B params in {res['quantize_ms']:.1f} ms; "
            f"fwd M=1 {res['m1']['ms']:.3f} ms ({res['m1']['GBps']:.0f} GB/s), "
            f"M=512 {res['m512']['ms']:.3f} ms ({res['m512']['TFLOPs']:.0f} TFLOP/s)")
        fu = res["fused"]
        log(f"[bench] 7B decoder, q|k|v and gate|up fused ({fu['launches_per_pass']} launches): "
            f"fwd M=1 {fu['m1']['ms']:.3f} ms ({fu['m1']['GBps']:.0f} GB/s), "
            f"M=512 {fu['m512']['ms']:.3f} ms ({fu['m512']['TFLOPs']:.0f} TFLOP/s)")
        torch.cuda.empty_cache()

    att = None
    if not args.no_attainable:
        att = bench_attainable(torch, fwd_bytes(1, N, K, r), copies, args.steps, args.warmup)
        log(f"[bench] attainable: empty kernel {att['empty_kernel_us']:.2f} us, plain read of the same bytes "
            f"{att['stream_same_bytes_us']:.2f} us ({att['stream_same_bytes_GBps']:.0f} GB/s), "
            f"1 GiB read {att['stream_1GiB_GBps']:.0f} GB/s")
        att["frac_of_stream_same_bytes"] = round(head["GBps"] / att["stream_same_bytes_GBps"], 4)
        att["frac_of_stream_1GiB"] = round(head["GBps"] / att["stream_1GiB_GBps"], 4)

    traffic = recorded_traffic("qlora_gemv_kernel_decode_4096x4096_m1.md", ["gemv.hip", "decode_common.h"])
    line = {
        "metric": METRIC,
        "value": round(head["GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_4096x4096_m1", "M": 1, "N": N, "K": K, "r": r, "alpha": 16.0,
                   "weight": "NF4 block 64 + E4M3 double quant block 256", "parallelism": "single GPU",
                   "cold_cache_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(head["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["hbm_frac"], 4), "traffic": traffic},
    }
    if att is not None:
        line["roofline"]["attainable"] = att
    if "train65b_22016x8192_m4096_fwd" in extra:
        f = extra["train65b_22016x8192_m4096_fwd"]
        line["m4096"] = {"workload": "train65b_22016x8192_m4096_fwd", "TFLOPs": round(f["TFLOPs"], 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "frac": round(f["mfma_frac"], 4), "ms": f["ms"]}
        if plain is not None:
            line["m4096"]["attainable"] = {**plain, "frac_of_it": round(f["TFLOPs"] / plain["TFLOPs"], 4)}
    if not args.no_cpu:
        log("[bench] cpu oracle baseline ...")
        line["cpu_baseline"] = cpu_baseline()
    line["extra"] = extra
    print(json.dumps(line))


if __name__ == "__main__":
    main()
