"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: values the
pages print (fixtures under tests/golden/ with their citations), closed forms,
brute force with exact rationals on tiny inputs, independent library routines
(mpmath, torch's bf16/E4M3 conversions, numpy fp32 division) and invariants.
The mutation tests at the end plant plausible mistakes in the oracle and check
that a pin catches each of them.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as o
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_numbers(name):
    vals = {}
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if len(parts) == 1:
                rows.append(float(parts[0]))
            else:
                vals[parts[0]] = float(parts[1])
    return rows, vals


# ---------------------------------------------------------------- NF4 table

def test_nf4_levels_match_printed_table():
    printed, _ = _golden_numbers("nf4_levels_printed.txt")
    L = o.nf4_levels_f64()
    assert len(printed) == 16
    # "to 4 decimals": every level within half a unit of the 4th decimal.  The
    # construction gives -0.0910499921 for the printed -0.0911, 7.9e-9 on the
    # other side of the -0.09105 rounding boundary, so the bound carries 1e-8.
    assert np.max(np.abs(L - np.array(printed))) <= 5e-5 + 1e-8
    # 15 of 16 agree under plain rounding; the 16th is the boundary case above
    assert int(np.sum(np.round(L, 4) == np.array(printed))) >= 15


def test_nf4_levels_structure():
    L = o.nf4_levels_f64()
    assert L[0] == -1.0 and L[15] == 1.0 and L[7] == 0.0
    assert np.all(np.diff(L) > 0)
    assert int(np.sum(L < 0)) == 7 and int(np.sum(L > 0)) == 8   # asymmetric, exact zero
    L32 = o.nf4_levels_f32()
    assert L32.dtype == np.float32 and L32[7] == 0.0


def test_nf4_levels_against_mpmath():
    """The same construction with 50-digit mpmath erfinv gives the same fp32 levels."""
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    mp.dps = 50
    off = mpmath.mpf("0.9677083")

    def q(count):
        return [mpmath.sqrt(2) * mpmath.erfinv(2 * (mpmath.mpf("0.5") + (off - mpmath.mpf("0.5")) * i / count) - 1)
                for i in range(1, count + 1)]

    vals = sorted([-v for v in q(7)] + [mpmath.mpf(0)] + q(8))
    mx = max(abs(v) for v in vals)
    ref = [v / mx for v in vals]
    L64 = o.nf4_levels_f64()
    for a, b in zip(L64, ref):
        assert abs(a - float(b)) < 1e-15
    ref32 = np.array([float(v) for v in ref]).astype(np.float32)
    # the fp64 values are far from fp32 rounding ties, so fp64->fp32 is safe here
    for v in ref:
        f = np.float32(float(v))
        up = np.nextafter(f, np.float32(np.inf))
        dn = np.nextafter(f, np.float32(-np.inf))
        if v != 0:
            gap = min(abs(float(v) - (float(f) + float(up)) / 2), abs(float(v) - (float(f) + float(dn)) / 2))
            assert gap > 1e-3 * float(up - f)
    assert np.array_equal(o.nf4_levels_f32().view(np.uint32), ref32.view(np.uint32))


# ---------------------------------------------------------------- quantize

def _brute_codes(w32, levels32):
    """Exact-rational nearest level of fp32(w / absmax) per 64-block, lowest index on ties."""
    Lf = [Fraction(float(v)) for v in levels32]
    zero_code = min(range(16), key=lambda i: (abs(Lf[i]), i))
    out = []
    for blk in w32.reshape(-1, 64):
        a = np.max(np.abs(blk))
        for w in blk:
            if a == 0:
                out.append(zero_code)
                continue
            x = Fraction(float(np.float32(w) / np.float32(a)))      # numpy IEEE fp32 division
            d = [abs(x - Lf[i]) for i in range(16)]
            out.append(min(range(16), key=lambda i: (d[i], i)))
    return np.array(out, dtype=np.uint8)


def test_quantize_matches_exact_bruteforce_random():
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((6, 128)) * rng.uniform(1e-3, 3, (6, 1))).astype(np.float32)
    W[2, :64] = 0.0                                   # an all-zero block
    W[3, 5] = -np.abs(W[3, :64]).max() * 2            # a negative block maximum
    codes, absmax = o.quantize_codes(W)
    assert np.array_equal(codes, _brute_codes(W, o.nf4_levels_f32()))
    assert np.array_equal(absmax, np.abs(W.reshape(-1, 64)).max(1))


@pytest.mark.parametrize("table", ["nf4", "uniform4", "fp4"])
def test_quantize_other_tables_match_exact_bruteforce(table):
    """Every table against exact-rational nearest level, with the quotients
    where fp64 distances alone cannot decide: tiny numbers between two levels of
    opposite sign (uniform 4-bit has no zero level, so +-1e-40 lie within one
    fp64 rounding of equidistant from +-1/15), signed zeros, exact midpoints,
    and FP4's duplicated zero."""
    L = {"nf4": o.nf4_levels_f32, "uniform4": o.uniform4_levels_f32, "fp4": o.fp4_levels_f32}[table]()
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    W[0, 0] = 1.0                                     # block max 1: quotients equal the weights
    special = [1e-40, -1e-40, 1e-45, -1e-45, 0.0, -0.0, 1e-30, -1e-30]
    special += [(float(L[j]) + float(L[j + 1])) / 2 for j in range(15) if L[j] != L[j + 1]]
    special = [np.float32(v) for v in special]
    W[0, 1:1 + len(special)] = special
    W[2, :64] = 0.0
    codes, _ = o.quantize_codes(W, L)
    assert np.array_equal(codes, _brute_codes(W, L))
    if table == "uniform4":
        assert codes[1] == 8 and codes[2] == 7        # +1e-40 -> +1/15, -1e-40 -> -1/15


def test_quantize_decision_boundaries():
    """Quotients exactly at, and one or two fp32 ulps around, every midpoint."""
    L = o.nf4_levels_f32()
    vals = []
    for j in range(15):
        m = (float(L[j]) + float(L[j + 1])) / 2        # exact in fp64
        f = np.float32(m)
        for k in range(-2, 3):
            g = f
            step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
            for _ in range(abs(k)):
                g = np.nextafter(g, step)
            vals.append(g)
    vals = np.array(vals, dtype=np.float32)
    pad = (-len(vals)) % 63
    vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 63)
    W = np.concatenate([np.ones((vals.shape[0], 1), np.float32), vals], axis=1)  # absmax 1 -> x == w
    codes, _ = o.quantize_codes(W)
    assert np.array_equal(codes, _brute_codes(W, L))
    # midpoints that are themselves fp32 numbers are exact ties -> the lower code
    ties = 0
    for j in range(15):
        m = (float(L[j]) + float(L[j + 1])) / 2
        if float(np.float32(m)) == m:
            ties += 1
            Wt = np.zeros((1, 64), np.float32)
            Wt[0, 0] = 1.0
            Wt[0, 1] = np.float32(m)
            c, _ = o.quantize_codes(Wt)
            assert c[1] == j
    assert ties == 5


def test_fp32_division_emulation_matches_ieee():
    rng = np.random.default_rng(5)
    a = rng.standard_normal(200000).astype(np.float32)
    b = np.abs(rng.standard_normal(200000)).astype(np.float32) + np.float32(1e-3)
    assert np.array_equal(o.f32(a.astype(np.float64) / b.astype(np.float64)), a / b)


def test_quantize_invariants():
    W = synth.normal_f32(21, (64, 256), 0.02)
    codes, absmax = o.quantize_codes(W)
    L = o.nf4_levels_f32().astype(np.float64)
    blocks = W.reshape(-1, 64)
    c = codes.reshape(-1, 64)
    for b in range(blocks.shape[0]):
        i = np.argmax(np.abs(blocks[b]))
        assert c[b, i] == (15 if blocks[b, i] > 0 else 0)
        assert L[c[b, i]] * absmax[b] == abs(blocks[b, i]) * np.sign(blocks[b, i])
    # re-quantizing the (pre-double-quant) dequantized block reproduces the codes
    deq = (L[codes] * np.repeat(absmax.astype(np.float64), 64)).astype(np.float32)
    codes2, _ = o.quantize_codes(deq.reshape(W.shape))
    assert np.array_equal(codes, codes2)
    # +-0 weights in a nonzero block map to the zero level
    Wz = W.copy()
    Wz[0, 3] = 0.0
    Wz[0, 4] = -0.0
    cz, _ = o.quantize_codes(Wz)
    assert cz[3] == 7 and cz[4] == 7


def test_pack_nibble_order():
    codes = np.arange(16, dtype=np.uint8)
    p = o.pack_nibbles(codes)
    assert list(p[:2]) == [0x10, 0x32]
    assert np.array_equal(o.unpack_nibbles(p), codes)


def test_worked_example_mae():
    """The pages' example: seed 0, N(0, 0.02), 4096*64 values, block 64."""
    _, g = _golden_numbers("worked_example.txt")
    w = np.random.default_rng(int(g["seed"])).normal(0, g["std"], size=int(g["count"]))
    w32 = w.astype(np.float32)
    for levels, key in ((o.nf4_levels_f32(), "mae_nf4"), (o.uniform4_levels_f32(), "mae_uniform4")):
        codes, a = o.quantize_codes(w32, levels)
        deq = levels.astype(np.float64)[codes] * np.repeat(a.astype(np.float64), 64)
        mae = np.abs(deq - w).mean()
        assert float("%.2e" % mae) == g[key], (key, mae)
    # full path: double-quantized constants and bf16 weights keep the NF4 figure
    W = w32.reshape(256, 1024)
    q = o.quantize_layer(W)
    wd = o.dequant_weight(q["codes"], q["c2"], q["c1"], q["mu"], 256, 1024)
    mae = np.abs(o.bf16_to_f64(wd).ravel() - w).mean()
    assert float("%.2e" % mae) == g["mae_nf4"]


def test_storage_overhead_closed_form():
    _, g = _golden_numbers("storage_overhead.txt")
    assert 32 / 64 == g["plain_bits"]
    shapes = [(256, 256), (4096, 4096), (11008, 4096), (4096, 11008), (22016, 8192)]
    for N, K in shapes:
        bits = o.storage_bits_per_param(N, K)
        assert round(bits, 3) == g["dq_bits"]
        assert abs(bits - (8 / 64 + 32 / (64 * 256)) - 32 / (N * K)) < 1e-12
    assert 8 / 64 + 32 / (64 * 256) == 0.126953125
    saved = 0.5 - (8 / 64 + 32 / (64 * 256))
    assert round(saved, 3) == g["saved_bits"]
    assert round(65e9 * saved / 8 / 1e9) == g["saved_gb_65b"]


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_definition():
    v = o.e4m3_value(np.arange(256))
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    fin = v[~np.isnan(v)]
    assert len(np.unique(fin)) == 253            # +0 and -0 collapse
    assert v[0x80] == 0.0 and np.signbit(v[0x80])


def test_e4m3_encode_matches_torch_and_bruteforce():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    mags = o.e4m3_value(np.arange(0x7F))
    mids = (mags[1:] + mags[:-1]) / 2                       # exact ties, fp32-representable
    t = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
        rng.standard_normal(5000) * 1e-3, mids, -mids, mags, -mags,
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
    ]).astype(np.float32)
    ours = o.e4m3_encode(t)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # saturation beyond the largest finite value
    big = np.array([448.0001, 470.0, 1e6, -500.0], np.float32)
    assert list(o.e4m3_encode(big)) == [0x7E, 0x7E, 0x7E, 0xFE]
    # brute force with exact rationals on a sample
    allv = [Fraction(float(m)) for m in mags]
    for x in t[::97]:
        a = Fraction(float(abs(x)))
        best = min(range(0x7F), key=lambda i: (abs(a - allv[i]), i & 1))
        code = best | (0x80 if np.signbit(x) else 0)
        assert o.e4m3_encode(np.array([x], np.float32))[0] == code


# ---------------------------------------------------------------- FP4 (E2M1) table

def _minifloat_by_code(exp_bits, man_bits, bias, specials):
    """Value of every bit pattern of a small binary float format, written from
    the general sign / biased exponent / fraction layout (None where the
    pattern is not a finite number).  specials: "ieee" (the top exponent is
    infinity and NaN), "fn" (only the all-ones pattern is NaN), "none"."""
    out = []
    top = (1 << exp_bits) - 1
    for code in range(1 << (1 + exp_bits + man_bits)):
        sign = -1 if code >> (exp_bits + man_bits) else 1
        e = (code >> man_bits) & top
        f = Fraction(code & ((1 << man_bits) - 1), 1 << man_bits)
        if (specials == "ieee" and e == top) or (specials == "fn" and e == top and f == 1 - Fraction(1, 1 << man_bits)):
            out.append(None)
            continue
        mag = f * Fraction(2) ** (1 - bias) if e == 0 else (1 + f) * Fraction(2) ** (e - bias)
        out.append(sign * mag)
    return out


def test_minifloat_enumerator_matches_torch_fp8():
    """The general enumerator above reproduces torch's two 8-bit float
    formats code by code, so it can stand as the reference for E2M1."""
    torch = pytest.importorskip("torch")
    for dtype, e, m, bias, sp in ((torch.float8_e4m3fn, 4, 3, 7, "fn"), (torch.float8_e5m2, 5, 2, 15, "ieee")):
        ref = torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()
        ours = _minifloat_by_code(e, m, bias, sp)
        for code in range(256):
            if ours[code] is None:
                assert not np.isfinite(ref[code]), (dtype, code)
            else:
                assert Fraction(float(ref[code])) == ours[code], (dtype, code)


def test_fp4_levels_from_e2m1_definition():
    """The FP4 table (reading: the E2M1 4-bit float) against the published
    E2M1 parameters (tests/golden/fp4_e2m1_format.txt) through the enumerator
    pinned on torch's fp8 formats: every bit pattern's value, sorted and
    divided by the largest magnitude; the two zeros at codes 7 and 8, both +0."""
    _, g = _golden_numbers("fp4_e2m1_format.txt")
    ref = _minifloat_by_code(int(g["exp_bits"]), int(g["man_bits"]), int(g["bias"]), "none")
    assert len(ref) == 16 and all(v is not None for v in ref)
    pos = sorted(v for v in ref if v > 0)
    assert max(pos) == Fraction(g["max_normal"]) and min(pos) == Fraction(g["min_subnormal"])
    assert min(v for v in pos if v >= 1) == Fraction(g["min_normal"])
    assert max(v for v in pos if v < Fraction(g["min_normal"])) == Fraction(g["max_subnormal"])
    top = max(abs(v) for v in ref)
    expect = np.array([float(v / top) for v in sorted(ref)], dtype=np.float64)
    expect[expect == 0.0] = 0.0
    L = o.fp4_levels_f32()
    assert L.dtype == np.float32 and len(L) == 16
    assert np.array_equal(L.view(np.uint32), expect.astype(np.float32).view(np.uint32))
    assert L.view(np.uint32)[7] == 0 and L.view(np.uint32)[8] == 0      # +0 twice
    assert np.all(np.diff(L) >= 0) and int(np.sum(np.diff(L) == 0)) == 1
    # the oracle's per-pattern decode agrees with the reference pattern by pattern
    assert all(Fraction(o.e2m1_value(b)) == ref[b] for b in range(16))


# ---------------------------------------------------------------- mean / double quant

def _check_rne(result, exact):
    r = np.float32(result)
    assert np.isfinite(r)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    d = abs(Fraction(float(r)) - exact)
    for nb in (up, dn):
        dn_ = abs(Fraction(float(nb)) - exact)
        assert d < dn_ or (d == dn_ and (r.view(np.uint32) & 1) == 0)


@pytest.mark.parametrize("case", range(7))
def test_mean_exact_rounding(case):
    rng = np.random.default_rng(100 + case)
    if case == 0:
        v = np.abs(rng.standard_normal(1000)).astype(np.float32) * 0.05
    elif case == 1:
        v = np.array([1e-45, 3e-45, 1e-40], np.float32)            # subnormals
    elif case == 2:
        v = np.array([3e38, 3e38, 1.0], np.float32)                 # the fp32 sum would overflow
    elif case == 3:
        v = np.array([0.1], np.float32)
    elif case == 4:
        v = np.zeros(17, np.float32)
    elif case == 5:
        v = np.array([1.0, np.float32(2 ** -24)], np.float32)       # a tie-like sum
    else:
        v = (np.abs(rng.standard_normal(3001)) * 10.0 ** rng.integers(-30, 30, 3001)).astype(np.float32)
    exact = sum(Fraction(float(x)) for x in v) / len(v)
    mu = o.mean_f32(v)
    assert o.exact_sum_f32(v) == sum(Fraction(float(x)) for x in v)
    _check_rne(mu, exact)


def test_round_rational_to_f32_against_float_path():
    rng = np.random.default_rng(8)
    for _ in range(2000):
        num = int(rng.integers(1, 2 ** 62))
        den = int(rng.integers(1, 2 ** 40))
        q = Fraction(num, den) * Fraction(2) ** int(rng.integers(-170, 60))
        _check_rne(o.round_rational_to_f32(q), q)


def test_double_quant_invariants():
    W = synth.normal_f32(0, (512, 4096), 0.02)
    absmax = o.blockwise_absmax(W)
    c2, c1, mu = o.double_quant(absmax)
    n = absmax.size
    assert c2.size == n and c1.size == -(-n // 256)
    x = o.f32(absmax.astype(np.float64) - float(mu))
    for b in range(c1.size):
        seg = x[b * 256:(b + 1) * 256]
        i = int(np.argmax(np.abs(seg)))
        assert c2[b * 256 + i] == (0x7E if seg[i] > 0 else 0xFE)   # block amax -> +-448
        assert c1[b] == np.float32(np.abs(seg).max() / 448.0)
    chat = o.dequant_constants(c2, c1, mu)
    # error of the constants is at most half an E4M3 step of the block's largest
    # centred value (1/28 of it) plus fp32 rounding
    amax_e = np.repeat(np.abs(np.pad(x, (0, (-n) % 256)).reshape(-1, 256)).max(1), 256)[:n]
    err = np.abs(chat.astype(np.float64) - absmax)
    assert np.all(err <= amax_e / 28 + 4 * np.spacing(absmax.astype(np.float32)))


def test_double_quant_centres_on_mean():
    """Constants with a large mean and a small spread keep a small error only if centred."""
    rng = np.random.default_rng(4)
    a = (1.0 + 0.1 * rng.random(4096)).astype(np.float32)
    c2, c1, mu = o.double_quant(a)
    chat = o.dequant_constants(c2, c1, mu)
    assert abs(float(mu) - float(np.mean(a.astype(np.float64)))) < 1e-6
    assert np.max(np.abs(chat.astype(np.float64) - a)) < 0.06 / 28 + 1e-6


def test_double_quant_constant_input_and_zero_weights():
    a = np.full(1000, 0.03125, np.float32)
    c2, c1, mu = o.double_quant(a)
    assert mu == np.float32(0.03125) and np.all(c1 == 0) and np.all(c2 == 0)
    assert np.all(o.dequant_constants(c2, c1, mu) == np.float32(0.03125))
    q = o.quantize_layer(np.zeros((8, 128), np.float32))
    assert np.all(q["codes"] == 0x77) and q["mu"] == 0 and np.all(q["c1"] == 0) and np.all(q["c2"] == 0)
    assert np.all(o.dequant_weight(q["codes"], q["c2"], q["c1"], q["mu"], 8, 128) == 0)


# ---------------------------------------------------------------- bf16 / dequant

def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-40, 38, 100000),
                        [0.0, -0.0, 1e-45, -3e-42, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]]).astype(np.float32)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.bf16_round(v), ref)


def test_dequant_weight_definition():
    W = synth.normal_f32(7, (12, 512), 0.02)
    q = o.quantize_layer(W)
    wd = o.dequant_weight(q["codes"], q["c2"], q["c1"], q["mu"], 12, 512)
    L = o.nf4_levels_f32().astype(np.float64)
    codes = o.unpack_nibbles(q["codes"]).reshape(12, 512)
    chat = o.dequant_constants(q["c2"], q["c1"], q["mu"]).reshape(12, 8)
    for n in range(12):
        for k in range(0, 512, 37):
            v = np.float32(L[codes[n, k]] * float(chat[n, k // 64]))
            b = np.float32(v).view(np.uint32)
            # bf16 nearest-even by integer rounding of the fp32 bit pattern
            expect = (int(b) + 0x7FFF + ((int(b) >> 16) & 1)) >> 16
            assert wd[n, k] == expect
    rows = np.array([3, 0, 11])
    assert np.array_equal(o.dequant_weight(q["codes"], q["c2"], q["c1"], q["mu"], 12, 512, rows=rows), wd[rows])
    # a 64-column slice quantized on its own has the same blocks, codes and W_deq columns
    for kb in (0, 5):
        sl = np.ascontiguousarray(W[:, 64 * kb:64 * kb + 64])
        codes_c, absmax_c = o.quantize_codes(sl)
        assert np.array_equal(absmax_c, q["absmax"].reshape(12, 8)[:, kb])
        assert np.array_equal(codes_c.reshape(12, 64), codes[:, 64 * kb:64 * kb + 64])
        cols = o.dequant_codes(codes_c.reshape(12, 64), chat[:, kb:kb + 1])
        assert np.array_equal(cols, wd[:, 64 * kb:64 * kb + 64])


# ---------------------------------------------------------------- forward / backward

def _tiny_layer(M=3, N=5, K=64, r=2, seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.02
    A = rng.standard_normal((r, K)) / K
    B = rng.standard_normal((N, r)) * 0.01
    dY = rng.standard_normal((M, N))
    return X, W, A, B, dY


def test_forward_against_loops():
    X, W, A, B, _ = _tiny_layer()
    s = 16 / 2
    Y, H = o.linear_fwd_f64(X, W, A, B, s)
    M, K = X.shape
    N, r = B.shape
    for m in range(M):
        h = [math.fsum(X[m, k] * A[j, k] for k in range(K)) for j in range(r)]
        for n in range(N):
            base = math.fsum(X[m, k] * W[n, k] for k in range(K))
            lora = math.fsum(h[j] * B[n, j] for j in range(r))
            assert abs(Y[m, n] - (base + s * lora)) < 1e-12


def test_forward_special_cases():
    X, W, A, B, _ = _tiny_layer(seed=1)
    Y, _ = o.linear_fwd_f64(X, W, A, np.zeros_like(B), 8.0)
    assert np.allclose(Y, X @ W.T, rtol=0, atol=1e-14)
    Y, _ = o.linear_fwd_f64(X, np.zeros_like(W), A, B, 8.0)
    assert np.allclose(Y, 8.0 * (X @ A.T) @ B.T, rtol=0, atol=1e-14)
    onehot = np.zeros((1, X.shape[1]))
    onehot[0, 9] = 1.0
    Y, _ = o.linear_fwd_f64(onehot, W, A, np.zeros_like(B), 8.0)
    assert np.array_equal(Y[0], W[:, 9])


def test_lora_scale():
    assert o.lora_scale(16, 8) == 2.0 and o.lora_scale(16, 64) == 0.25 and o.lora_scale(16, 16) == 1.0


def test_backward_finite_differences():
    X, W, A, B, dY = _tiny_layer(M=2, N=3, K=64, r=2, seed=2)
    s = 3.0
    g = o.linear_bwd_f64(dY, X, W, A, B, s)

    def loss(Xv, Av, Bv):
        Y, _ = o.linear_fwd_f64(Xv, W, Av, Bv, s)
        return float(np.sum(dY * Y))

    h = 1e-3
    for name, arr in (("dX", X), ("dA", A), ("dB", B)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy()
            p[idx] += h
            m_ = arr.copy()
            m_[idx] -= h
            args_p = {"dX": (p, A, B), "dA": (X, p, B), "dB": (X, A, p)}[name]
            args_m = {"dX": (m_, A, B), "dA": (X, m_, B), "dB": (X, A, m_)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        scale = np.max(np.abs(num)) + 1e-30
        assert np.max(np.abs(num - g[name])) <= 1e-7 * scale, name
    assert np.allclose(g["dH"], s * dY @ B) and np.allclose(g["H"], X @ A.T)


def test_bits_wrappers_use_exact_bf16_values():
    d = synth.make_layer(synth.SINGLE, with_dy=True)
    q = o.quantize_layer(d["W"])
    wd = o.dequant_weight(q["codes"], q["c2"], q["c1"], q["mu"], 256, 256)
    Y, H = o.linear_fwd(d["X"], wd, d["A"], d["B"], 16.0, 8)
    Y2, _ = o.linear_fwd_f64(synth.bf16_bits_to_f32(d["X"]).astype(np.float64),
                             synth.bf16_bits_to_f32(wd).astype(np.float64),
                             synth.bf16_bits_to_f32(d["A"]).astype(np.float64),
                             synth.bf16_bits_to_f32(d["B"]).astype(np.float64), 2.0)
    assert np.array_equal(Y, Y2)


# ---------------------------------------------------------------- planted mistakes

def test_planted_mistakes_are_caught(monkeypatch):
    """Plausible slips in the oracle each fail one of the pins above."""
    # 1. levels built with symmetric 8/8 quantiles (no exact zero) -> structure pin
    import oracle.qlora_oracle as qo
    real_levels = qo.nf4_levels_f64

    def sym_levels(offset=qo.NF4_OFFSET):
        p = 0.5 + (offset - 0.5) * np.arange(1, 9) / 8
        v = np.sort(np.concatenate([-qo.ndtri(p), qo.ndtri(p)]))
        return v / np.abs(v).max()

    monkeypatch.setattr(qo, "nf4_levels_f64", sym_levels)
    with pytest.raises(AssertionError):
        test_nf4_levels_structure()
    monkeypatch.setattr(qo, "nf4_levels_f64", real_levels)

    # 2. double quant without mean centring -> centring pin
    real_mean = qo.mean_f32
    monkeypatch.setattr(qo, "mean_f32", lambda v: np.float32(0.0))
    with pytest.raises(AssertionError):
        test_double_quant_centres_on_mean()
    monkeypatch.setattr(qo, "mean_f32", real_mean)

    # 3. a dropped LoRA term in the backward dX -> finite differences
    real_bwd = qo.linear_bwd_f64

    def bad_bwd(dY, X, W, A, B, s):
        g = real_bwd(dY, X, W, A, B, s)
        g["dX"] = dY @ W
        return g

    monkeypatch.setattr(o, "linear_bwd_f64", bad_bwd)
    with pytest.raises(AssertionError):
        test_backward_finite_differences()
    monkeypatch.setattr(o, "linear_bwd_f64", real_bwd)

    # 4. a transposed LoRA product in the forward -> the loop pin
    real_fwd = qo.linear_fwd_f64

    def bad_fwd2(X, W, A, B, s):
        H = X @ A.T
        return X @ W.T + s * (H[:, ::-1] @ B.T), H

    monkeypatch.setattr(o, "linear_fwd_f64", bad_fwd2)
    with pytest.raises(AssertionError):
        test_forward_against_loops()
    monkeypatch.setattr(o, "linear_fwd_f64", real_fwd)

    # 5. ties to the upper level in the nearest-level search -> boundary pin
    real_near = qo._nearest_level

    def upper_ties(x32, levels32):
        d = np.abs(x32.astype(np.float64)[..., None] - levels32.astype(np.float64)[None, :])
        return (15 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)

    monkeypatch.setattr(qo, "_nearest_level", upper_ties)
    with pytest.raises(AssertionError):
        test_quantize_decision_boundaries()
    monkeypatch.setattr(qo, "_nearest_level", real_near)


def test_planted_mistakes_in_code_tables_and_merge_are_caught(monkeypatch):
    """A wrong E2M1 magnitude, a subnormal read with an implicit leading one,
    and the merge rounded through fp32 before bf16 each fail their pin."""
    import oracle.qlora_oracle as qo
    real_e2m1 = qo.e2m1_value

    def wrong_top(bits):
        return 5.0 * (-1 if bits & 8 else 1) if bits & 7 == 7 else real_e2m1(bits)

    def implicit_one(bits):
        v = real_e2m1(bits)
        return v + (-1.0 if bits & 8 else 1.0) if (bits >> 1) & 3 == 0 else v

    for bad in (wrong_top, implicit_one):
        monkeypatch.setattr(qo, "e2m1_value", bad)
        with pytest.raises(AssertionError):
            test_fp4_levels_from_e2m1_definition()
    monkeypatch.setattr(qo, "e2m1_value", real_e2m1)

    real_merge = qo.merge_weight

    def via_fp32(Wdeq_bits, A_bits, B_bits, alpha, r):
        s = np.float64(qo.lora_scale(alpha, r))
        A = qo.bf16_to_f64(A_bits).reshape(r, -1)
        B = qo.bf16_to_f64(B_bits).reshape(-1, r)
        W = qo.bf16_to_f64(Wdeq_bits).reshape(B.shape[0], A.shape[1])
        acc = np.zeros_like(W)
        for j in range(r):
            acc = acc + B[:, j:j + 1] * A[j:j + 1, :]
        return qo.bf16_round(qo.f32(W + s * acc))

    monkeypatch.setattr(o, "merge_weight", via_fp32)
    with pytest.raises(AssertionError):
        test_merge_weight_against_exact_rational_rounding()
    monkeypatch.setattr(o, "merge_weight", real_merge)


def test_bf16_weight_quantization_is_the_widened_fp32_quantization():
    """A bf16 weight quantizes as the fp32 number it widens to: known bit
    patterns decode to their values (1, -1, 0.5, the smallest subnormal, -0),
    and on random weights the result equals quantize_layer of the widened
    values computed through fp64."""
    import oracle
    probe = np.array([0x3F80, 0xBF80, 0x3F00, 0x0001, 0x8000] + [0] * 59, np.uint16).reshape(1, 64)
    q = oracle.quantize_layer_bf16(probe)
    assert q["absmax"][0] == np.float32(1.0)
    codes = oracle.unpack_nibbles(q["codes"]).reshape(-1)
    assert list(codes[:5]) == [15, 0, int(np.argmin(np.abs(oracle.nf4_levels_f32() - 0.5))), 7, 7]
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    bits = oracle.bf16_round(W)
    widened = oracle.bf16_to_f64(bits).astype(np.float32)
    a, b = oracle.quantize_layer_bf16(bits), oracle.quantize_layer(widened)
    for k in ("codes", "absmax", "c2", "c1"):
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k
    assert np.float32(a["mu"]).tobytes() == np.float32(b["mu"]).tobytes()


def _bf16_rne_exact(v):
    """bf16 bits of the rational v rounded to nearest, ties to even (reference
    by rational arithmetic)."""
    from fractions import Fraction
    import math
    v = Fraction(v)
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # 2^e <= a < 2^(e+1)
    ulp = Fraction(2) ** (max(e, -126) - 7)
    q = a / ulp
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = float(n * ulp)
    return sign | (int(np.float32(val).view(np.uint32)) >> 16)


def test_bf16_round_f64_matches_rational_rounding():
    """One-step fp64 -> bf16 rounding against rational round-to-nearest-even on
    random values, exact halfway points (both parities), bf16 subnormals and
    values one fp64 ulp either side of a halfway point."""
    import oracle
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(400) * np.exp2(rng.integers(-140, 20, 400)))
    for bits in (0x3F80, 0x3F81, 0x4049, 0x0003, 0x0080, 0xBF83):
        lo = float(np.uint32(bits << 16).view(np.float32))
        hi = float(np.uint32((bits + 1) << 16).view(np.float32))
        mid = (lo + hi) / 2                       # exact in fp64
        vals += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), -mid]
    vals = np.array(vals, dtype=np.float64)
    got = oracle.bf16_round_f64(vals)
    exp = np.array([_bf16_rne_exact(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, exp)


def test_merge_weight_special_cases_and_exact_sums():
    """Merged weight: B = 0 gives W_deq itself; with s a power of two and
    operands whose fp64 sums are exact, the result is the rational W + s B A
    rounded once to bf16."""
    import oracle
    from fractions import Fraction
    rng = np.random.default_rng(9)
    N, K, r, alpha = 6, 16, 8, 16.0                # s = 2
    def bf(x):
        return oracle.bf16_round(np.asarray(x, np.float32))
    Wb = bf(rng.uniform(-1, 1, (N, K)) * 0.05)
    Ab = bf(rng.uniform(0.25, 1, (r, K)) * rng.choice([-1, 1], (r, K)))
    Bb = bf(rng.uniform(0.25, 1, (N, r)) * rng.choice([-1, 1], (N, r)) * 2.0 ** -6)
    assert np.array_equal(oracle.merge_weight(Wb, Ab, np.zeros_like(Bb), alpha, r), Wb)
    got = oracle.merge_weight(Wb, Ab, Bb, alpha, r)
    W, A, B = (oracle.bf16_to_f64(x) for x in (Wb, Ab, Bb))
    s = Fraction(oracle.lora_scale(alpha, r))
    assert s == 2
    for n in range(N):
        for k in range(K):
            v = Fraction(W[n, k]) + s * sum(Fraction(B[n, j]) * Fraction(A[j, k]) for j in range(r))
            assert got[n, k] == _bf16_rne_exact(v), (n, k)


def _bf16_tie_distance(v):
    """Distance of the rational v from the nearest bf16 rounding midpoint."""
    import math
    a = abs(Fraction(v))
    if a == 0:
        return Fraction(1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 7)
    q = a / ulp
    return abs((q - math.floor(q)) - Fraction(1, 2)) * ulp


def _merge_exact(Wb, Ab, Bb, alpha, r):
    """bf16 bits of W + s sum_j B A in rational arithmetic, one rounding, with a
    mask of the elements that lie within 2^-40 (relative) of a bf16 midpoint."""
    W, A, B = (o.bf16_to_f64(x) for x in (Wb, Ab, Bb))
    s = Fraction(o.lora_scale(alpha, r))
    N, K = W.shape
    out = np.zeros((N, K), np.uint16)
    near = np.zeros((N, K), bool)
    for n in range(N):
        for k in range(K):
            v = Fraction(W[n, k]) + s * sum(Fraction(B[n, j]) * Fraction(A[j, k]) for j in range(r))
            out[n, k] = _bf16_rne_exact(v)
            near[n, k] = _bf16_tie_distance(v) <= Fraction(2) ** -40 * abs(v)
    return out, near


def test_merge_weight_against_exact_rational_rounding():
    """merge_weight on random bf16 operands whose sums are not exact in fp64
    (s = fp32(16/6) is not a power of two) equals W + s B A computed in
    rational arithmetic and rounded once to bf16, except where the exact value
    lies within 2^-40 of a bf16 midpoint (there the fp64 summation order may
    decide); and on operands built to sit just off a midpoint, where rounding
    through fp32 first would land on the midpoint and round the other way."""
    rng = np.random.default_rng(21)

    def bf(x):
        return o.bf16_round(np.asarray(x, np.float32))

    N, K, r, alpha = 12, 64, 6, 16.0
    Wb = bf(rng.standard_normal((N, K)) * 0.02)
    Ab = bf(rng.standard_normal((r, K)) / K)
    Bb = bf(rng.standard_normal((N, r)) * 0.01)
    got = o.merge_weight(Wb, Ab, Bb, alpha, r)
    exp, near = _merge_exact(Wb, Ab, Bb, alpha, r)
    assert int(near.sum()) < N * K // 100
    assert np.array_equal(got[~near], exp[~near])

    # s = 1 (alpha = r = 2): W = +-1, B A = 2^-8 + 2^-30 (just above the
    # midpoint between 1 and 1 + 2^-7), exactly 2^-8 (a tie: to even), 3 2^-8
    # (a tie: to even, upwards), and 2^-8 - 2^-30 (just below)
    one, e8, e15 = 0x3F80, 0x3B80, 0x3800
    Wb = np.array([[one] * 4, [0xBF80] * 4], np.uint16)
    Ab = np.array([[0x3F80, 0x3F80, 0x4040, 0x3F80], [e15, 0, 0, 0xB800]], np.uint16)
    Bb = np.array([[e8, e15], [0xBB80, 0xB800]], np.uint16)
    got = o.merge_weight(Wb, Ab, Bb, 2.0, 2)
    exp, near = _merge_exact(Wb, Ab, Bb, 2.0, 2)
    # columns 1 and 2 are exact midpoints; every sum here is exact in fp64
    assert not near[:, [0, 3]].any() and near[:, [1, 2]].all()
    assert list(exp[0]) == [0x3F81, 0x3F80, 0x3F82, 0x3F80]
    assert np.array_equal(got, exp)


# ---------------------------------------------------------------- the parity tolerance itself

def test_check_close_bf16_floor():
    """Half a bf16 ulp at powers of two and between them; and a rank-one
    output rounded exactly to bf16 passes only with the floor (its own rounding
    exceeds 2e-2 * RMS), while a real error of 3e-2 * RMS still fails."""
    from gpu_util import bf16_f64, check_close, half_ulp_bf16
    v = np.array([1.0, 1.5, 0.75, -2.0, 0.0, 2.0 ** -130])
    assert np.array_equal(half_ulp_bf16(v), [2.0 ** -8, 2.0 ** -8, 2.0 ** -9, 2.0 ** -7, 0.0, 2.0 ** -138])
    rng = np.random.default_rng(5)
    u, w = rng.standard_normal(300), rng.standard_normal(1024)
    u[0], w[0] = 4.5, 4.4                       # a large corner element: max/RMS ~ 20
    ref = np.outer(u, w)
    got = bf16_f64(o.bf16_round_f64(ref))
    rms = np.linalg.norm(ref) / np.sqrt(ref.size)
    assert np.max(np.abs(got - ref)) / rms > 2e-2       # the output's own rounding misses the bar
    with pytest.raises(AssertionError):
        check_close(got, ref, "rank one")
    check_close(got, ref, "rank one", bf16_floor=True)
    bad = got.copy()
    bad[1, 1] += 3e-2 * rms + half_ulp_bf16(ref[1, 1])
    with pytest.raises(AssertionError):
        check_close(bad, ref, "rank one", bf16_floor=True)
    # "auto": the floor applies here, where the exactly rounded output misses
    # the bar, and a real error beyond it still fails ...
    check_close(got, ref, "rank one", bf16_floor="auto")
    with pytest.raises(AssertionError):
        check_close(bad, ref, "rank one", bf16_floor="auto")
    # ... but not on a full-rank output, whose rounded values meet the plain
    # rule: an error of 2.5e-2 x RMS (within half an ulp of a large element
    # plus the bar) fails there without the floor
    full = rng.standard_normal((300, 1024))
    rms_f = np.linalg.norm(full) / np.sqrt(full.size)
    got_f = bf16_f64(o.bf16_round_f64(full))
    check_close(got_f, full, "full rank", bf16_floor="auto")
    k = np.unravel_index(np.argmax(np.abs(full)), full.shape)
    off = got_f.copy()
    off[k] = full[k] + 2.5e-2 * rms_f
    assert abs(off[k] - full[k]) - half_ulp_bf16(full[k]) < 2e-2 * rms_f   # the floor would hide it
    with pytest.raises(AssertionError):
        check_close(off, full, "full rank", bf16_floor="auto")
