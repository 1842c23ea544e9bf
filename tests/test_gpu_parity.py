"""GPU parity: libqlora.so (through the C ABI) against the CPU oracle.

Integer and byte results (packed codes, absmax, c2, c1, the mean, the bf16
dequantized weight) must match bit for bit.  Floating-point layer outputs
(Y, H, dX, dA, dB) must meet the tolerance in gpu_util (relative Frobenius
error <= 5e-3, max error <= 2e-2 x RMS).  Every input comes from the seeded
generators in ``synth``; every expected value comes from ``oracle``.
"""

import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_f64, check_close, dev_bf16, dev_f32, host, host_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - the GPU suite needs an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import bit_nf4_quantized_quant_amd as qa  # noqa: E402  (raises if libqlora.so is missing)

qa.lib()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_quantize(W):
    q = qa.quantize(dev_f32(W))
    torch.cuda.synchronize()
    return q


def check_quantized(q, ref, rows=None):
    N, K = q.N, q.K
    codes = host(q.codes)
    if rows is None:
        assert np.array_equal(codes, ref["codes"]), "packed codes differ"
    else:
        assert np.array_equal(codes[rows], ref["codes"]), "packed codes differ (sampled rows)"
    assert np.array_equal(host(q.absmax).view(np.uint32), ref["absmax"].view(np.uint32)), "absmax differs"
    assert host(q.mean).view(np.uint32)[0] == np.float32(ref["mu"]).view(np.uint32), \
        f"mean differs: {host(q.mean)[0]!r} vs {ref['mu']!r}"
    assert np.array_equal(host(q.c1).view(np.uint32)[:ref["c1"].size], ref["c1"].view(np.uint32)), "c1 differs"
    assert np.array_equal(host(q.c2), ref["c2"]), "c2 differs"


def special_weight(N, K, seed):
    """N(0, 0.02) weights plus the degenerate cases of blockwise NF4."""
    W = synth.normal_f32(seed, (N, K), 0.02)
    L = oracle.nf4_levels_f32()
    W[0, :64] = 0.0                                      # all-zero block -> code 7, absmax 0
    if K >= 128:
        W[0, 64] = 1.0                                   # block max 1: quotients equal the weights
        mids = [(float(L[j]) + float(L[j + 1])) / 2 for j in range(15)]
        exact = [np.float32(m) for m in mids if float(np.float32(m)) == m]
        W[0, 65:65 + len(exact)] = exact                 # exact ties -> lower level
        W[0, 80] = -0.0
        W[0, 81] = np.float32(1e-40)                     # fp32 subnormal
    if N > 1:
        W[1, :64] = -np.abs(W[1, :64])                   # negative block maximum
        W[1, 5] = np.float32(3e30)                       # huge outlier
    return W


# ------------------------------------------------------------------ quantize / double quant / dequant

@pytest.mark.parametrize("N,K", [(256, 256), (1, 64), (5, 192), (17, 1024), (300, 832)])
def test_quantize_and_double_quant_bitexact(N, K):
    say(f"[quantize] N={N} K={K}")
    W = special_weight(N, K, seed=N * 7 + K)
    ref = oracle.quantize_layer(W)
    check_quantized(gpu_quantize(W), ref)


def test_quantize_decode_layer_bitexact():
    say("[quantize] decode layer 4096x4096")
    W = synth.normal_f32(synth.SEED_W, (4096, 4096), 0.02)
    check_quantized(gpu_quantize(W), oracle.quantize_layer(W))


def test_quantize_constant_constants_and_zero_weight():
    # every block has the same absmax -> centred constants are all 0 -> c1 = 0, c2 = 0
    W = np.zeros((8, 256), np.float32)
    W[:, ::64] = 0.5
    ref = oracle.quantize_layer(W)
    assert np.all(ref["c1"] == 0)
    check_quantized(gpu_quantize(W), ref)
    Z = np.zeros((4, 128), np.float32)
    check_quantized(gpu_quantize(Z), oracle.quantize_layer(Z))


@pytest.mark.parametrize("N,K", [(256, 256), (5, 192), (300, 832)])
def test_quantize_bf16_weights_bitexact(N, K):
    """bf16 base weights (normal ~0.02 rounded to bf16, an all-zero block and
    a block of subnormals): codes and every constant bit-exact with the
    oracle's quantization of the widened values."""
    say(f"[quantize bf16] N={N} K={K}")
    bits = oracle.bf16_round(special_weight(N, K, seed=3 * N + K))
    bits[0, :64] = 0
    if N > 1:
        bits[1, :64] = np.arange(1, 65, dtype=np.uint16)     # subnormal bf16 values
    ref = oracle.quantize_layer_bf16(bits)
    Wd = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    check_quantized(qa.quantize(Wd), ref)


def test_quantize_quotients_at_midpoints_and_bucket_edges():
    """Quotients exactly at, and up to 3 fp32 ulps around, every midpoint of
    adjacent levels and every multiple of 1/16 in [-1, 1] (the edges of the
    kernel's threshold buckets): blocks whose absmax is exactly 1, so each
    quotient is the weight itself; codes bit-exact with the oracle."""
    say("[quantize] quotients at midpoints and bucket edges")
    L = oracle.nf4_levels_f32().astype(np.float64)
    centres = list((L[:-1] + L[1:]) / 2) + [q / 16 - 1 for q in range(33)]
    probes = []
    for c in centres:
        up = dn = np.float32(c)
        probes.append(up)
        for _ in range(3):
            up = np.nextafter(up, np.float32(2))
            dn = np.nextafter(dn, np.float32(-2))
            probes += [up, dn]
    probes = np.array([v for v in probes if -1 <= v <= 1], np.float32)
    nblk = -(-len(probes) // 63)
    nblk += (-nblk) % 4                       # 4 blocks per row
    flat = np.zeros(nblk * 63, np.float32)
    flat[:len(probes)] = probes
    W = np.zeros((nblk, 64), np.float32)
    W[:, 0] = np.where(np.arange(nblk) % 2 == 0, 1.0, -1.0)   # absmax exactly 1
    W[:, 1:] = flat.reshape(nblk, 63)
    W = W.reshape(nblk // 4, 256)
    check_quantized(gpu_quantize(W), oracle.quantize_layer(W))


@pytest.mark.parametrize("N,K,r", [(256, 256, 8), (5, 192, 16), (300, 832, 72), (33, 1088, 128), (70, 64, 1),
                                   (9, 128, 0)])
def test_merge_bitexact(N, K, r):
    """Merged weight W_deq + s B A (bf16) bit-exact with the oracle's fp64
    definition; ragged row counts, r from 0 to 128."""
    say(f"[merge] N={N} K={K} r={r}")
    d = synth.make_layer(synth.LayerShape("t", M=1, N=N, K=K, r=max(r, 1), seed_offset=17 * N + K + r))
    ref = oracle.quantize_layer(d["W"])
    wd = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K)
    alpha = 16.0
    if r > 0:
        exp = oracle.merge_weight(wd, d["A"][:r], d["B"][:, :r], alpha, r)
        A, B = dev_bf16(np.ascontiguousarray(d["A"][:r])), dev_bf16(np.ascontiguousarray(d["B"][:, :r]))
    else:
        exp, A, B = wd, None, None
    got = host_bf16_bits(qa.merge(gpu_quantize(d["W"]), A, B, alpha))
    assert np.array_equal(got, exp)


TABLES = [(1, "uniform4"), (2, "fp4")]


def table_levels(table):
    return {0: oracle.nf4_levels_f32, 1: oracle.uniform4_levels_f32, 2: oracle.fp4_levels_f32}[table]()


@pytest.mark.parametrize("table,name", TABLES, ids=[t[1] for t in TABLES])
def test_code_tables_quantize_dequant_merge_bitexact(table, name):
    """The uniform 4-bit and FP4 tables through the same kernels: codes,
    constants, the dequantized weight (fp32 and bf16 input) and the merge
    bit-exact with the oracle run on the same table."""
    say(f"[table {name}] quantize / dequant / merge")
    L = table_levels(table)
    N, K, r = 33, 1088, 16
    W = special_weight(N, K, seed=700 + table)
    ref = oracle.quantize_layer(W, L)
    q = qa.quantize(dev_f32(W), table=table)
    check_quantized(q, ref)
    wd = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K, levels32=L)
    assert np.array_equal(host_bf16_bits(qa.dequantize(q)), wd)
    bits = oracle.bf16_round(W)
    check_quantized(qa.quantize(dev_bf16(bits), table=table), oracle.quantize_layer_bf16(bits) if table == 0
                    else oracle.quantize_layer((bits.astype(np.uint32) << 16).view(np.float32), L))
    d = synth.make_layer(synth.LayerShape("t", M=1, N=N, K=K, r=r, seed_offset=800 + table))
    exp = oracle.merge_weight(wd, d["A"], d["B"], 16.0, r)
    assert np.array_equal(host_bf16_bits(qa.merge(q, dev_bf16(d["A"]), dev_bf16(d["B"]), 16.0)), exp)


@pytest.mark.parametrize("table,name", TABLES, ids=[t[1] for t in TABLES])
@pytest.mark.parametrize("M,N,K,r", [(1, 300, 1024, 16), (7, 129, 512, 24), (130, 300, 448, 72),
                                     (520, 600, 1280, 32), (70, 130, 192, 16)])
def test_code_tables_forward_backward(table, name, M, N, K, r):
    """Forward (GEMV, matrix-core decode and tiled paths) and backward (both
    dX paths) with the other code tables, against the oracle on the same
    table."""
    say(f"[table {name}] M={M} N={N} K={K} r={r}")
    L = table_levels(table)
    d = synth.make_layer(synth.LayerShape("t", M=M, N=N, K=K, r=r, seed_offset=900 + table * 31 + M), with_dy=True)
    ref = oracle.quantize_layer(d["W"], L)
    wd = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K, levels32=L)
    q = qa.quantize(dev_f32(d["W"]), table=table)
    X, A, B, dY = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"]), dev_bf16(d["dY"])
    Y, H = qa.linear_fwd(X, q, A, B, 16.0)
    dX, dA, dB = qa.linear_bwd(dY, X, q, A, B, 16.0, H=H)
    torch.cuda.synchronize()
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], 16.0, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y")
    g = oracle.linear_bwd(d["dY"], d["X"], wd, d["A"], d["B"], 16.0, r)
    check_close(bf16_f64(host_bf16_bits(dX)), g["dX"], "dX")
    check_close(bf16_f64(host_bf16_bits(dA)), g["dA"], "dA", bf16_floor=True if M == 1 else "auto")
    check_close(bf16_f64(host_bf16_bits(dB)), g["dB"], "dB", bf16_floor=True if M == 1 else "auto")


def test_saved_weight_reloads_to_the_same_layer(tmp_path):
    """A quantized weight written to .npz and read back onto the GPU gives the
    same W_deq and the same forward output, bit for bit."""
    d = synth.make_layer(synth.LayerShape("t", M=3, N=130, K=320, r=8, seed_offset=5151))
    q = gpu_quantize(d["W"])
    path = str(tmp_path / "w.npz")
    qa.save_quantized(q, path)
    q2 = qa.load_quantized(path, device="cuda")
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    assert torch.equal(qa.dequantize(q).view(torch.int16), qa.dequantize(q2).view(torch.int16))
    Y1, _ = qa.linear_fwd(X, q, A, B, 16.0)
    Y2, _ = qa.linear_fwd(X, q2, A, B, 16.0)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


@pytest.mark.parametrize("N,K", [(256, 256), (5, 192), (33, 1088)])
def test_dequant_bitexact(N, K):
    W = special_weight(N, K, seed=3 * N + K)
    W[1, 5] = 0.1
    q = gpu_quantize(W)
    ref = oracle.quantize_layer(W)
    wd = qa.dequantize(q)
    torch.cuda.synchronize()
    exp = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K)
    assert np.array_equal(host_bf16_bits(wd), exp)


def test_e4m3_decode_every_code():
    """Each finite E4M3 byte dequantizes to its exact value (level 1.0, c1 = 1, mean 0)."""
    codes8 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    N, K = codes8.size, 64
    packed = torch.full((N, K // 2), 0xFF, dtype=torch.uint8, device="cuda")   # code 15 = +1.0
    c2 = torch.from_numpy(codes8).cuda()
    c1 = torch.ones(1, dtype=torch.float32, device="cuda")
    mean = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    qa.qlora_nf4_dequant(packed, c2, c1, mean, N, K, out)
    torch.cuda.synchronize()
    got_bits = host_bf16_bits(out)
    got = bf16_f64(got_bits)
    exp = oracle.e4m3_value(codes8)
    assert np.array_equal(got[:, 0], exp) and np.all(got == got[:, :1])
    # bit patterns too, through the oracle's own dequantization (-0 * 1 + 0 = +0)
    ref = oracle.dequant_weight(np.full((N, K // 2), 0xFF, np.uint8), codes8, np.ones(1, np.float32),
                                np.float32(0.0), N, K)
    assert np.array_equal(got_bits, ref)


# ------------------------------------------------------------------ forward

def oracle_layer(d, alpha, r):
    ref = oracle.quantize_layer(d["W"])
    N, K = d["W"].shape
    wd = oracle.dequant_weight(ref["codes"], ref["c2"], ref["c1"], ref["mu"], N, K)
    return ref, wd


def run_fwd(d, q, alpha, r, ws=None):
    """One forward; also checks that no bounded wait of the launch gave up."""
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    if ws is None:
        ws = qa.fwd_workspace(X.shape[0], q.N, q.K, r, "cuda")
    before = qa.fwd_wait_count(ws)
    Y, H = qa.linear_fwd(X, q, A, B, alpha, workspace=ws)
    torch.cuda.synchronize()
    assert qa.fwd_wait_count(ws) == before, "a wait for a partial result gave up"
    return Y, H


FWD_CASES = [
    # M, N, K, r   (decode path for M <= 16, tiled MFMA path above)
    (16, 256, 256, 8), (1, 256, 256, 8), (4, 100, 320, 5), (3, 33, 64, 1), (16, 130, 192, 128),
    (2, 300, 1024, 16), (7, 129, 512, 24), (1, 1000, 2048, 64), (5, 77, 768, 12), (16, 64, 4096, 64),
    (1, 96, 11008, 64), (12, 40, 1280, 40),
    (17, 130, 192, 16), (33, 257, 128, 1), (130, 300, 448, 72), (256, 512, 1024, 64), (64, 64, 64, 64),
    (600, 700, 1536, 16), (513, 2304, 512, 64),
    # larger M: 128 x 128 tiles with split-K, a ragged M and r, one whole
    # round of 256 x 256 tiles
    (1024, 300, 448, 72), (1100, 600, 1280, 33), (2048, 8192, 256, 8),
    # 16 x 18 tiles of 256: one whole round on 256 x 256 tiles and a ragged
    # tail of 296 columns, on 256 x 256 tiles split in two along K (K = 128),
    # or on 128 x 128 tiles where K = 64 leaves a single step
    (4096, 4392, 128, 16), (4096, 4392, 64, 16),
]


@pytest.mark.parametrize("M,N,K,r", FWD_CASES)
def test_forward_parity(M, N, K, r):
    say(f"[fwd] M={M} N={N} K={K} r={r}")
    shape = synth.LayerShape("t", M=M, N=N, K=K, r=r, seed_offset=M * 1000 + N + K + r)
    d = synth.make_layer(shape)
    alpha = 16.0
    ref, wd = oracle_layer(d, alpha, r)
    q = gpu_quantize(d["W"])
    Y, H = run_fwd(d, q, alpha, r)
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y")
    check_close(host(H), Hr, "H")


def test_forward_special_cases():
    M, N, K, r = 16, 192, 256, 8
    for Mx in (M, 40):
        d = synth.make_layer(synth.LayerShape("t", M=Mx, N=N, K=K, r=r, seed_offset=77 + Mx))
        # B = 0: the plain dequantized product
        d0 = dict(d, B=np.zeros_like(d["B"]))
        ref, wd = oracle_layer(d0, 16.0, r)
        Y, _ = run_fwd(d0, gpu_quantize(d0["W"]), 16.0, r)
        Yr = bf16_f64(d0["X"]) @ bf16_f64(wd).T
        check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y (B=0)")
        # W = 0: codes 7, constants 0 -> exactly the LoRA branch s (X A^T) B^T
        dz = dict(d, W=np.zeros_like(d["W"]))
        Y, _ = run_fwd(dz, gpu_quantize(dz["W"]), 16.0, r)
        Yr = 2.0 * (bf16_f64(d["X"]) @ bf16_f64(d["A"]).T) @ bf16_f64(d["B"]).T
        check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y (W=0)")


def test_forward_one_hot_rows_select_weight_columns():
    """One-hot X rows with B = 0 reproduce columns of the dequantized weight."""
    N, K, r = 128, 256, 8
    for M in (4, 32, 64):
        d = synth.make_layer(synth.LayerShape("t", M=M, N=N, K=K, r=r, seed_offset=5 + M))
        X = np.zeros((M, K), np.float32)
        cols = (np.arange(M) * 37) % K
        X[np.arange(M), cols] = 1.0
        d = dict(d, X=synth.f32_to_bf16_bits(X), B=np.zeros_like(d["B"]))
        ref, wd = oracle_layer(d, 16.0, r)
        Y, _ = run_fwd(d, gpu_quantize(d["W"]), 16.0, r)
        got = host_bf16_bits(Y).astype(np.int32)
        exp = wd[:, cols].T.astype(np.int32)
        if M > 16:
            assert np.array_equal(got, exp)          # tiled path multiplies the exact bf16 W_deq
        else:
            # the decode path scales hi+lo bf16 levels in fp32 after the product, so a
            # value lying within 2^-17 of a bf16 rounding boundary may land one ulp over
            assert np.max(np.abs(got - exp)) <= 1


def shared_workspace(shapes):
    """One zeroed forward workspace large enough for every (M, N, K, r)."""
    need = max(qa.qlora_linear_fwd_workspace(*sh) for sh in shapes)
    return torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")


def test_forward_deterministic_and_workspace_reusable():
    """Repeated calls give identical bits, and one workspace serves any mix of
    shapes, ranks and layers without adapter (r = 0)."""
    shapes = ((1, 512, 512, 16), (16, 512, 512, 16), (64, 512, 512, 16), (3, 2048, 1024, 72),
              (1, 100, 128, 8), (2, 512, 512, 0), (16, 2048, 1024, 72), (5, 300, 256, 0))
    ws = shared_workspace(shapes)
    layers = {}
    for M, N, K, r in shapes:
        d = synth.make_layer(synth.LayerShape("t", M=M, N=N, K=K, r=r, seed_offset=900 + M + N + r))
        layers[(M, N, K, r)] = (d, gpu_quantize(d["W"]))
    first = {}
    for rep in range(3):
        for key, (d, q) in layers.items():
            r = key[3]
            A, B = adapter(d, r)
            Y, H = qa.linear_fwd(dev_bf16(d["X"]), q, A, B, 16.0, workspace=ws)
            torch.cuda.synchronize()
            if rep == 0:
                first[key] = (Y, H)
                _, wd = oracle_layer(d, 16.0, max(r, 1))
                if r:
                    Yr, _ = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], 16.0, r)
                else:
                    Yr, _ = oracle.linear_fwd_f64(bf16_f64(d["X"]), bf16_f64(wd), np.zeros((0, key[2])),
                                                  np.zeros((key[1], 0)), 0.0)
                check_close(bf16_f64(host_bf16_bits(Y)), Yr, f"Y {key}")
            else:
                assert torch.equal(Y.view(torch.int16), first[key][0].view(torch.int16)), key
                assert (H is None) == (r == 0)
                if r:
                    assert torch.equal(H, first[key][1]), key
    # the decode kernels' bounded waits never gave up
    assert qa.fwd_wait_count(ws) == 0


def test_forward_graph_replay_matches_oracle_and_eager():
    """The mode the benchmark times: many forwards captured in one HIP graph,
    rotating over weight copies, all sharing one workspace.  52 calls (M = 1,
    4, 16 and 64 interleaved, 4 weight copies, each call its own X and Y),
    replayed three times with eager work and synchronizations between the
    replays; every Y of every replay equals the eager result bit for bit and
    meets the tolerance against the oracle, and no wait gave up."""
    N, K, r, alpha, copies = 1024, 1024, 16, 16.0, 4
    layers = []
    for c in range(copies):
        d = synth.make_layer(synth.LayerShape("t", M=1, N=N, K=K, r=r, seed_offset=4400 + c))
        _, wd = oracle_layer(d, alpha, r)
        layers.append((d, wd, gpu_quantize(d["W"]), dev_bf16(d["A"]), dev_bf16(d["B"])))
    Ms = (1, 4, 16, 64)
    calls = []
    for i in range(52):
        M = Ms[i % 4]
        xb = synth.f32_to_bf16_bits(synth.normal_f32(5000 + i, (M, K), 1.0))
        calls.append((i % copies, xb, dev_bf16(xb), torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
    ws = shared_workspace([(M, N, K, r) for M in Ms])

    def run_all():
        for c, _, X, Y in calls:
            _, _, q, A, B = layers[c]
            qa.qlora_linear_fwd(X, q.codes, q.c2, q.c1, q.mean, A, B, alpha, Y, None, ws, N)

    run_all()                                   # eager reference
    torch.cuda.synchronize()
    eager = [Y.clone() for *_, Y in calls]
    for (c, xb, _, _), Ye in zip(calls, eager):
        d, wd = layers[c][0], layers[c][1]
        Yr, _ = oracle.linear_fwd(xb, wd, d["A"], d["B"], alpha, r)
        check_close(bf16_f64(host_bf16_bits(Ye)), Yr, f"Y eager copy {c} M={xb.shape[0]}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run_all()
    torch.cuda.synchronize()
    for rep in range(3):
        for *_, Y in calls:
            Y.fill_(0)                          # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((c, xb, _, Y), Ye) in enumerate(zip(calls, eager)):
            assert torch.equal(Y.view(torch.int16), Ye.view(torch.int16)), (rep, i)
    assert qa.fwd_wait_count(ws) == 0


@pytest.mark.parametrize("M", [1, 8])
def test_forward_wait_gives_up_and_stays_correct(M):
    """Forced from the host: launch counters of the workspace are set 5
    launches ahead of the others, so some workgroups never see the tag they
    wait for on the published partials.  At M = 1 (GEMV) the LoRA-down
    counters move ahead of the weight counters: the weight workgroups never
    see this launch's H.  At M = 8 (matrix-core path) half of the weight
    counters move ahead: workgroups on different counters disagree on the
    launch, so H partials and the K slices' exchanged products go missing.
    Every wait reaches its deadline (about 1 ms), the waiting lanes compute
    their values themselves, every kernel ends normally, Y and H still match
    the oracle, and the wait counter says the fallback ran.  (Counter layout:
    eight 64-bit weight counters 128 bytes apart from byte 128, eight
    LoRA-down counters from byte 1280.)"""
    N, K, r, alpha = 512, 1024, 16, 16.0
    d = synth.make_layer(synth.LayerShape("t", M=M, N=N, K=K, r=r, seed_offset=4500 + M))
    _, wd = oracle_layer(d, alpha, r)
    q = gpu_quantize(d["W"])
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    ws = qa.fwd_workspace(M, N, K, r, "cuda")
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    Y, H = qa.linear_fwd(X, q, A, B, alpha, workspace=ws)     # one consistent launch first
    torch.cuda.synchronize()
    assert qa.fwd_wait_count(ws) == 0
    first, slots = (1280, range(8)) if M <= 4 else (128, range(4))
    for s in slots:
        ctr = ws[first + 128 * s:first + 128 * s + 8].view(torch.int64)
        ctr += 5 << 20
    torch.cuda.synchronize()
    say(f"[wait give-up] M={M}: launching with desynchronized counters")
    for rep in range(2):
        Y, H = qa.linear_fwd(X, q, A, B, alpha, workspace=ws)
        torch.cuda.synchronize()
        check_close(bf16_f64(host_bf16_bits(Y)), Yr, f"Y after give-up, launch {rep}")
        check_close(host(H), Hr, f"H after give-up, launch {rep}")
    assert qa.fwd_wait_count(ws) > 0
    qa.clear_fwd_wait_count(ws)
    torch.cuda.synchronize()
    assert qa.fwd_wait_count(ws) == 0


@pytest.mark.parametrize("shape", synth.DECODE, ids=lambda sh: sh.name)
def test_forward_decode_layer_full_size(shape):
    """The 4096 x 4096 decode layer at M = 1, 4, 16: every output against the oracle."""
    say(f"[fwd full] {shape.name}")
    d = synth.make_layer(shape)
    ref, wd = oracle_layer(d, shape.alpha, shape.r)
    q = gpu_quantize(d["W"])
    check_quantized(q, ref)
    Y, H = run_fwd(d, q, shape.alpha, shape.r)
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], shape.alpha, shape.r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y")
    check_close(host(H), Hr, "H")


# ------------------------------------------------------------------ backward

# dX runs on 128 x 128 tiles with split-K here (520 x 600 and 512 x 130 with M >= 512: N % 8
# == 0 and not, so 16-byte and element-wise dY loads); the 65B-scale test below takes 256 x 256
# tiles.  dH and dB come from the single pass over dY where M, N and r are multiples of 8 and
# r <= 64: 16 x 256 (two 128-column chunks per workgroup), 520 x 600 (four chunks, ragged last
# row tile and column block), 200 x 1032 (r = 24: ragged rows, columns and rank), 64 x 136
# (a chunk of 8 columns), 640 x 22016 (two row tiles per workgroup), 2112 x 4096 (33 row
# tiles over 32 workgroups along M) and 136 x 1000 (r = 56: the second 32-wide rank tile
# partly used); the others take the three separate products.
BWD_CASES = [(16, 256, 256, 8), (3, 100, 320, 5), (70, 130, 192, 16), (257, 300, 448, 72), (1, 64, 64, 1),
             (520, 600, 1280, 32), (512, 130, 320, 8), (200, 1032, 192, 24), (64, 136, 128, 64),
             (640, 22016, 64, 64), (2112, 4096, 64, 16), (136, 1000, 128, 56)]


@pytest.mark.parametrize("M,N,K,r", BWD_CASES)
def test_backward_parity(M, N, K, r):
    say(f"[bwd] M={M} N={N} K={K} r={r}")
    shape = synth.LayerShape("t", M=M, N=N, K=K, r=r, seed_offset=31 * M + N + K + r)
    d = synth.make_layer(shape, with_dy=True)
    alpha = 16.0
    ref, wd = oracle_layer(d, alpha, r)
    g = oracle.linear_bwd(d["dY"], d["X"], wd, d["A"], d["B"], alpha, r)
    q = gpu_quantize(d["W"])
    X, A, B, dY = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"]), dev_bf16(d["dY"])
    _, H = qa.linear_fwd(X, q, A, B, alpha)
    for Hin in (H, None):
        dX, dA, dB = qa.linear_bwd(dY, X, q, A, B, alpha, H=Hin)
        torch.cuda.synchronize()
        check_close(bf16_f64(host_bf16_bits(dX)), g["dX"], "dX")
        check_close(bf16_f64(host_bf16_bits(dA)), g["dA"], "dA", bf16_floor=True if M == 1 else "auto")
        check_close(bf16_f64(host_bf16_bits(dB)), g["dB"], "dB", bf16_floor=True if M == 1 else "auto")
    _, dA2, dB2 = qa.linear_bwd(dY, X, q, A, B, alpha, H=H, want_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dA2.view(torch.int16), dA.view(torch.int16))
    assert torch.equal(dB2.view(torch.int16), dB.view(torch.int16))


def test_backward_no_outputs_gives_zero_input_grads():
    """N = 0: the sums over the output dimension are empty, so dX = 0 and dA = 0."""
    M, K, r = 40, 128, 8
    d = synth.make_layer(synth.LayerShape("t", M=M, N=1, K=K, r=r, seed_offset=4343))
    q = qa.QuantizedWeight(0, K, torch.zeros((1, K // 2), dtype=torch.uint8, device="cuda"), None,
                           torch.zeros(1, dtype=torch.uint8, device="cuda"),
                           torch.zeros(1, dtype=torch.float32, device="cuda"),
                           torch.zeros(1, dtype=torch.float32, device="cuda"))
    X = dev_bf16(d["X"])
    dY = torch.zeros((M, 0), dtype=torch.bfloat16, device="cuda")
    A = dev_bf16(d["A"])
    B = torch.zeros((0, r), dtype=torch.bfloat16, device="cuda")
    dX, dA, dB = qa.linear_bwd(dY, X, q, A, B, 16.0)
    torch.cuda.synchronize()
    assert dB.numel() == 0
    assert float(dX.float().abs().sum()) == 0.0 and float(dA.float().abs().sum()) == 0.0


def test_backward_empty_batch_gives_zero_lora_grads():
    N, K, r = 64, 128, 8
    d = synth.make_layer(synth.LayerShape("t", M=1, N=N, K=K, r=r, seed_offset=4242))
    q = gpu_quantize(d["W"])
    X = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros((0, N), dtype=torch.bfloat16, device="cuda")
    A, B = dev_bf16(d["A"]), dev_bf16(d["B"])
    dX, dA, dB = qa.linear_bwd(dY, X, q, A, B, 16.0)
    torch.cuda.synchronize()
    assert dX.numel() == 0
    assert float(dA.float().abs().sum()) == 0.0 and float(dB.float().abs().sum()) == 0.0


# ------------------------------------------------------------------ no adapter (r = 0)

NOADAPTER_CASES = [(1, 256, 256), (16, 300, 512), (40, 130, 192), (300, 257, 320)]


@pytest.mark.parametrize("M,N,K", NOADAPTER_CASES)
def test_no_adapter_forward_and_backward(M, N, K):
    """r = 0: Y = X W_deq^T and dX = dY W_deq, with A and B passed as NULL."""
    say(f"[r=0] M={M} N={N} K={K}")
    d = synth.make_layer(synth.LayerShape("t", M=M, N=N, K=K, r=1, seed_offset=7 * M + N + K), with_dy=True)
    _, wd = oracle_layer(d, 16.0, 1)
    q = gpu_quantize(d["W"])
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    Y, H = qa.linear_fwd(X, q, None, None, 16.0)
    dX, dA, dB = qa.linear_bwd(dY, X, q, None, None, 16.0)
    torch.cuda.synchronize()
    assert H is None and dA is None and dB is None
    Xf, Wf, dYf = bf16_f64(d["X"]), bf16_f64(wd), bf16_f64(d["dY"])
    no_a, no_b = np.zeros((0, K)), np.zeros((N, 0))
    Yr, _ = oracle.linear_fwd_f64(Xf, Wf, no_a, no_b, 0.0)
    g = oracle.linear_bwd_f64(dYf, Xf, Wf, no_a, no_b, 0.0)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y (r=0)")
    check_close(bf16_f64(host_bf16_bits(dX)), g["dX"], "dX (r=0)")


# ------------------------------------------------------------------ full-size layers, sampled outputs

def oracle_sampled(W, rows, col_block=None):
    """The oracle's quantization of a full-size weight: every constant (absmax,
    c2, c1, mean) in full, codes and W_deq only for the sampled rows and, if
    asked, for one 64-column block of every row."""
    N, K = W.shape
    absmax = oracle.blockwise_absmax(W)
    c2, c1, mu = oracle.double_quant(absmax)
    chat = oracle.dequant_constants(c2, c1, mu).reshape(N, K // 64)
    codes_r, _ = oracle.quantize_codes(W[rows])
    out = {"absmax": absmax, "c2": c2, "c1": c1, "mu": mu,
           "codes": oracle.pack_nibbles(codes_r).reshape(len(rows), K // 2),
           "wd_rows": oracle.dequant_codes(codes_r.reshape(len(rows), K), chat[rows])}
    if col_block is not None:
        kb = col_block
        codes_c, _ = oracle.quantize_codes(np.ascontiguousarray(W[:, 64 * kb:64 * kb + 64]))
        out["wd_cols"] = oracle.dequant_codes(codes_c.reshape(N, 64), chat[:, kb:kb + 1])
    return out


def adapter(d, r):
    return (dev_bf16(d["A"]), dev_bf16(d["B"])) if r > 0 else (None, None)


def check_fwd_sampled(d, ref, rows, Y, H, alpha, r, name, msel=None):
    X = d["X"] if msel is None else d["X"][msel]
    Yg = bf16_f64(host_bf16_bits(Y))[:, rows] if msel is None else bf16_f64(host_bf16_bits(Y))[msel][:, rows]
    if r > 0:
        Yr, Hr = oracle.linear_fwd(X, ref["wd_rows"], d["A"], d["B"][rows], alpha, r)
        Hg = host(H) if msel is None else host(H)[msel]
        check_close(Hg, Hr, f"H {name}")
    else:
        Yr, _ = oracle.linear_fwd_f64(bf16_f64(X), bf16_f64(ref["wd_rows"]), np.zeros((0, X.shape[1])),
                                      np.zeros((len(rows), 0)), 0.0)
    check_close(Yg, Yr, f"Y {name}")


MLP_SHAPES = [("gate_up_11008x4096", 11008, 4096), ("down_4096x11008", 4096, 11008)]


@pytest.mark.parametrize("name,N,K", MLP_SHAPES, ids=[s[0] for s in MLP_SHAPES])
def test_forward_mlp_layer_full_size_sampled(name, N, K):
    """Llama-7B-shaped MLP projections at M = 1, 16, 256 (decode and tiled
    paths) in the launch configuration the benchmark uses; all constants and
    512 sampled output columns against the oracle."""
    shapes = [sh for sh in synth.MLP if sh.N == N and sh.K == K]
    rows = np.sort(np.random.default_rng(N + K).choice(N, 512, replace=False))
    d0 = synth.make_layer(shapes[0])
    ref = oracle_sampled(d0["W"], rows)
    q = gpu_quantize(d0["W"])
    check_quantized(q, ref, rows)
    for sh in shapes:
        say(f"[mlp full] {sh.name}")
        d = synth.make_layer(sh)
        assert np.array_equal(d["W"], d0["W"])
        A, B = adapter(d, sh.r)
        Y, H = qa.linear_fwd(dev_bf16(d["X"]), q, A, B, sh.alpha)
        torch.cuda.synchronize()
        check_fwd_sampled(d, ref, rows, Y, H, sh.alpha, sh.r, sh.name)


@pytest.mark.parametrize("M,N", [(1, 16400), (4, 9000)])
def test_forward_gemv_32_row_tiles_every_output(M, N):
    """The GEMV on 32-row tiles, which it takes when 16-row tiles would need
    three or more rounds of resident workgroups and 32-row tiles fewer (M = 1,
    N = 16400: 1089 workgroups become 577, the last tile 16 rows; M = 4, one
    workgroup per CU, N = 9000: 627 become 346, the last tile 8 rows; K =
    2048: one piece per lane over all of K), every output of Y and H against
    the oracle."""
    K, r, alpha = 2048, 64, 16.0
    say(f"[gemv 32-row tiles] M={M} N={N} K={K} r={r}")
    shape = synth.LayerShape("t32r", M=M, N=N, K=K, r=r, seed_offset=9100 + M)
    d = synth.make_layer(shape)
    _, wd = oracle_layer(d, alpha, r)
    q = gpu_quantize(d["W"])
    Y, H = run_fwd(d, q, alpha, r)
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y (32-row GEMV tiles)")
    check_close(host(H), Hr, "H (32-row GEMV tiles)")


def test_forward_256_tiles_every_output():
    """A forward that runs on 256 x 256 tiles (M = 1000, N = 16320: 4 x 64
    tiles, one per CU, the last row and column tiles ragged), every output
    of Y and H against the oracle."""
    M, N, K, r, alpha = 1000, 16320, 1024, 64, 16.0
    say(f"[fwd 256 tiles] M={M} N={N} K={K} r={r}")
    shape = synth.LayerShape("t256", M=M, N=N, K=K, r=r, seed_offset=9001)
    d = synth.make_layer(shape)
    _, wd = oracle_layer(d, alpha, r)
    q = gpu_quantize(d["W"])
    Y, H = qa.linear_fwd(dev_bf16(d["X"]), q, dev_bf16(d["A"]), dev_bf16(d["B"]), alpha)
    torch.cuda.synchronize()
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y (256 x 256 tiles)")
    check_close(host(H), Hr, "H (256 x 256 tiles)")


def test_forward_256_tiles_split_tail_every_output():
    """A forward whose 256 x 256 tiles leave a partial last round (M = 512,
    N = 33040: 2 x 130 tiles on 256 CUs): the columns of the whole round run
    in one launch and the 272-column tail on 256 x 256 tiles split in two
    along the reduction (K = 576: 5 and 4 steps; the last tile 16 columns
    wide), reduced into Y's tail columns.  Every output of Y and H against
    the oracle."""
    M, N, K, r, alpha = 512, 33040, 576, 64, 16.0
    say(f"[fwd split tail] M={M} N={N} K={K} r={r}")
    shape = synth.LayerShape("t256t", M=M, N=N, K=K, r=r, seed_offset=9003)
    d = synth.make_layer(shape)
    _, wd = oracle_layer(d, alpha, r)
    q = gpu_quantize(d["W"])
    Y, H = qa.linear_fwd(dev_bf16(d["X"]), q, dev_bf16(d["A"]), dev_bf16(d["B"]), alpha)
    torch.cuda.synchronize()
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y (split tail)")
    check_close(bf16_f64(host_bf16_bits(Y))[:, 32768:], Yr[:, 32768:], "Y (tail columns)")
    check_close(host(H), Hr, "H (split tail)")


STREAM_K_CASES = [
    # (M, N, K, r): 128 x 128 tiles whose split-K plan (two pieces per tile)
    # needs more than one round of resident workgroups (two per CU on 256
    # CUs), so the steps are shared out stream-K, at least 32 per workgroup
    (1000, 4200, 4032, 16),  # 8 x 33 tiles of 63 steps: 32.5 per workgroup; last row and column tiles 104 wide
    (600, 6600, 4096, 8),    # 5 x 52 tiles of 64 steps: 32.5 per workgroup; last tiles 88 rows, 72 columns
]


@pytest.mark.parametrize("M,N,K,r", STREAM_K_CASES)
def test_forward_stream_k_every_output(M, N, K, r):
    """Forwards on 128 x 128 tiles whose steps are shared out stream-K (each
    workgroup a contiguous run of steps across tile boundaries, shared tiles
    summed from their pieces in step order): every output of Y and H against
    the oracle, and the same Y again from a second call on the same
    workspace."""
    alpha = 16.0
    say(f"[fwd stream-K] M={M} N={N} K={K} r={r}")
    shape = synth.LayerShape("tsk", M=M, N=N, K=K, r=r, seed_offset=9100 + M)
    d = synth.make_layer(shape)
    _, wd = oracle_layer(d, alpha, r)
    q = gpu_quantize(d["W"])
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    ws = qa.fwd_workspace(M, N, K, r, "cuda")
    Y, H = qa.linear_fwd(X, q, A, B, alpha, workspace=ws)
    Y2, _ = qa.linear_fwd(X, q, A, B, alpha, workspace=ws)
    torch.cuda.synchronize()
    Yr, Hr = oracle.linear_fwd(d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(Y)), Yr, "Y (stream-K)")
    check_close(host(H), Hr, "H (stream-K)")
    assert np.array_equal(host_bf16_bits(Y), host_bf16_bits(Y2)), "second call on the same workspace differs"


def test_backward_256_tiles_every_output():
    """A backward whose dX runs on 256 x 256 tiles (M = 1000, K = 16384: 4 x 64
    tiles) with a ragged reduction (N = 1004: 15 full steps and 44 rows, dY
    read element-wise since N % 8 != 0), every output of dX, dA and dB
    against the oracle."""
    M, N, K, r, alpha = 1000, 1004, 16384, 16, 16.0
    say(f"[bwd 256 tiles] M={M} N={N} K={K} r={r}")
    shape = synth.LayerShape("t256b", M=M, N=N, K=K, r=r, seed_offset=9002)
    d = synth.make_layer(shape, with_dy=True)
    _, wd = oracle_layer(d, alpha, r)
    q = gpu_quantize(d["W"])
    X, A, B, dY = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"]), dev_bf16(d["dY"])
    dX, dA, dB = qa.linear_bwd(dY, X, q, A, B, alpha)
    torch.cuda.synchronize()
    g = oracle.linear_bwd(d["dY"], d["X"], wd, d["A"], d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(dX)), g["dX"], "dX (256 x 256 tiles)")
    check_close(bf16_f64(host_bf16_bits(dA)), g["dA"], "dA")
    check_close(bf16_f64(host_bf16_bits(dB)), g["dB"], "dB")


def test_train65b_layer_full_size_sampled():
    """The 65B-scale training layer (W 22016 x 8192, M = 4096, r = 64) forward
    and backward: all constants, sampled rows of W_deq, sampled outputs of Y,
    dX (one 64-column block of every row), dA (the same columns) and dB (sampled
    rows) against the oracle."""
    sh = synth.TRAIN65B
    M, N, K, r, alpha = sh.M, sh.N, sh.K, sh.r, sh.alpha
    say(f"[65b] generating {sh.name}")
    d = synth.make_layer(sh, with_dy=True)
    rng = np.random.default_rng(65)
    rows = np.sort(rng.choice(N, 128, replace=False))
    kb = int(rng.integers(K // 64))
    msel = np.sort(rng.choice(M, 256, replace=False))
    ref = oracle_sampled(d["W"], rows, kb)
    say("[65b] gpu")
    q = gpu_quantize(d["W"])
    check_quantized(q, ref, rows)
    X, dY = dev_bf16(d["X"]), dev_bf16(d["dY"])
    A, B = adapter(d, r)
    Y, H = qa.linear_fwd(X, q, A, B, alpha)
    dX, dA, dB = qa.linear_bwd(dY, X, q, A, B, alpha, H=H)
    torch.cuda.synchronize()
    del X, dY
    say("[65b] forward check")
    check_fwd_sampled(d, ref, rows, Y, H, alpha, r, "65b", msel=msel)
    say("[65b] backward check")
    cols = slice(64 * kb, 64 * kb + 64)
    g1 = oracle.linear_bwd(d["dY"], np.ascontiguousarray(d["X"][:, cols]), ref["wd_cols"],
                           np.ascontiguousarray(d["A"][:, cols]), d["B"], alpha, r)
    check_close(bf16_f64(host_bf16_bits(dX))[:, cols], g1["dX"], "dX (64-column block)")
    check_close(bf16_f64(host_bf16_bits(dA))[:, cols], g1["dA"], "dA (64-column block)")
    g2 = oracle.linear_bwd(np.ascontiguousarray(d["dY"][:, rows]), d["X"], ref["wd_rows"], d["A"],
                           d["B"][rows], alpha, r)
    check_close(bf16_f64(host_bf16_bits(dB))[rows], g2["dB"], "dB (sampled rows)")


def test_decoder_fused_qkv_full_size_sampled():
    """The decoder's q|k|v group as one 12288 x 4096 weight with the
    block-structured rank-32 adapter (q rows on columns 0..15, v rows on
    16..31, k rows zero), at M = 1 and M = 512: constants in full and 256
    sampled output columns spread over the three segments, against the
    oracle; also at M = 12 and 16, where the matrix-core decode kernel runs
    on two K slices (the grid of four would need a second round)."""
    N, K, r = 12288, 4096, 32
    rows = np.sort(np.concatenate([np.random.default_rng(77 + i).choice(4096, 85 + (i == 0), replace=False) + 4096 * i
                                   for i in range(3)]))
    q = ref = None
    for M in (1, 12, 16, 512):
        sh = synth.LayerShape(f"decoder_qkv_m{M}", M=M, N=N, K=K, r=r, seed_offset=1777)
        say(f"[decoder fused] {sh.name}")
        d = synth.make_layer(sh)
        d["B"] = np.where(synth.fused_qkv_b_mask(N, r), d["B"], np.uint16(0))
        if q is None:
            ref = oracle_sampled(d["W"], rows)
            q = gpu_quantize(d["W"])
            check_quantized(q, ref, rows)
        A, B = adapter(d, r)
        Y, H = qa.linear_fwd(dev_bf16(d["X"]), q, A, B, synth.FUSED_QKV_ALPHA)
        torch.cuda.synchronize()
        check_fwd_sampled(d, ref, rows, Y, H, synth.FUSED_QKV_ALPHA, r, sh.name)


def test_decode_slices_past_one_round_sampled():
    """The matrix-core decode kernel where the slice model's grid would need
    several rounds of workgroups (22016 x 4096: 344 row groups, two slices
    of 32 blocks, the operands loaded straight from memory), M = 5, 8 and 16:
    constants in full and 256 sampled output columns against the oracle, no
    bounded wait giving up."""
    N, K, r, alpha = 22016, 4096, 64, 16.0
    rows = np.sort(np.random.default_rng(4242).choice(N, 256, replace=False))
    q = ref = None
    for M in (5, 8, 16):
        sh = synth.LayerShape(f"slices_m{M}", M=M, N=N, K=K, r=r, seed_offset=4242)
        say(f"[decode slices] {sh.name}")
        d = synth.make_layer(sh)
        if q is None:
            ref = oracle_sampled(d["W"], rows)
            q = gpu_quantize(d["W"])
            check_quantized(q, ref, rows)
        Y, H = run_fwd(d, q, alpha, r)
        check_fwd_sampled(d, ref, rows, Y, H, alpha, r, sh.name)


@pytest.mark.parametrize("layer", [0, synth.DECODER_LAYERS - 1])
def test_decoder_layer_full_size_sampled(layer):
    """One layer of the 7B-shaped decoder (q, k, v, o, gate, up, down; LoRA
    r = 16 on q and v only) at M = 1 and M = 512: all constants and 256 sampled
    output columns per linear against the oracle."""
    for mi, (mod, N, K, r) in enumerate(synth.DECODER_MODULES):
        seed = synth.decoder_seed(layer, mi)
        rows = np.sort(np.random.default_rng(seed).choice(N, 256, replace=False))
        q = ref = None
        for M in (1, 512):
            sh = synth.LayerShape(f"decoder_l{layer}_{mod}_m{M}", M=M, N=N, K=K, r=r, seed_offset=seed)
            say(f"[decoder] {sh.name}")
            d = synth.make_layer(sh)
            if q is None:
                ref = oracle_sampled(d["W"], rows)
                q = gpu_quantize(d["W"])
                check_quantized(q, ref, rows)
            A, B = adapter(d, r)
            Y, H = qa.linear_fwd(dev_bf16(d["X"]), q, A, B, sh.alpha)
            torch.cuda.synchronize()
            check_fwd_sampled(d, ref, rows, Y, H, sh.alpha, r, sh.name)
