"""CPU oracle for the QLoRA NF4 linear layer (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and
it shares no code, table or constant with the GPU library: the NF4 code table
is rebuilt here from its definition, every rounding point is written out from
the format definitions, and only the seeded input generators in ``synth`` feed
both sides.

Sources (page title, then the section the step follows):
  * itwiki "QLoRA", section 4-bit NormalFloat (NF4): the 16-level code built
    from N(0,1) quantiles with an exact zero, blockwise absmax quantization
    with block 64, nearest-level coding, dequantization as level * absmax,
    and the worked MAE example.
  * itwiki "QLoRA", section double quantization: the absmax constants are
    mean-centred and quantized symmetrically to an 8-bit float in blocks of
    256 with one fp32 constant per block; the storage-overhead formula.
  * itwiki "QLoRA", section on the computation: the layer output is
    X * doubleDequant(c1, c2, W) + X * L1 * L2 in bf16, with gradients only for
    the input and the LoRA factors.
  * minnong511 "quantization", the boxed equation y = W x + (alpha/r) B A x
    and the backward notes (W frozen, A and B get gradients).
  * kdkrkwhr "LoRA vs Q-LoRA", section 1: B is d x r, A is r x k.

Arithmetic model.  Everything is computed in fp64.  Each fp32 operation of the
specification is emulated as the fp64 result of the same operation on the fp32
operands, rounded once to fp32; for +, -, *, / this equals the IEEE fp32
result, because fp64 carries more than 2*24+2 bits.  bf16 and E4M3 roundings
are written from their format definitions.  Matrix products are plain fp64
numpy products of the exact bf16 operand values.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
from scipy.special import ndtri

F64 = np.float64
F32 = np.float32

NF4_OFFSET = 0.9677083   # bitsandbytes' offset as printed on the itwiki page
BLOCK = 64               # NF4 block size (weights per absmax constant)
DQ_BLOCK = 256           # double-quant block size (constants per fp32 constant)
E4M3_MAX = 448.0


def f32(x) -> np.ndarray:
    """Round fp64 values to the nearest fp32 (ties to even)."""
    return np.asarray(x, dtype=F64).astype(F32)


# ---------------------------------------------------------------------------
# NF4 code table (itwiki "QLoRA", NF4 section)
# ---------------------------------------------------------------------------

def nf4_levels_f64(offset: float = NF4_OFFSET) -> np.ndarray:
    """The 16 NF4 levels in fp64, sorted ascending.

    The positive half takes the standard-normal quantiles of 8 probabilities
    evenly spaced between 0.5 (excluded) and ``offset``; the negative half takes
    the negated quantiles of 7 such probabilities; an exact 0 sits between them.
    The set is divided by its largest magnitude, so the ends are -1 and +1.
    """
    def quantiles(count: int) -> np.ndarray:
        steps = np.arange(1, count + 1, dtype=F64)
        probs = 0.5 + (offset - 0.5) * steps / count
        return ndtri(probs)

    levels = np.concatenate([-quantiles(7), np.zeros(1), quantiles(8)])
    levels = np.sort(levels)
    return levels / np.max(np.abs(levels))


def nf4_levels_f32(offset: float = NF4_OFFSET) -> np.ndarray:
    return f32(nf4_levels_f64(offset))


def uniform4_levels_f32() -> np.ndarray:
    """The comparison grid of the worked example: 16 evenly spaced levels on [-1, 1]."""
    return f32(np.linspace(-1.0, 1.0, 16))


E2M1_EXP_BITS, E2M1_MAN_BITS, E2M1_BIAS = 2, 1, 1   # the 4-bit float format (E2M1)


def e2m1_value(bits: int) -> float:
    """Value of a 4-bit float bit pattern: sign, 2 exponent bits with bias 1,
    1 mantissa bit; exponent field 0 is subnormal (0 or 0.5); no infinity or
    NaN encodings."""
    sign = -1.0 if (bits >> (E2M1_EXP_BITS + E2M1_MAN_BITS)) & 1 else 1.0
    e = (bits >> E2M1_MAN_BITS) & ((1 << E2M1_EXP_BITS) - 1)
    m = bits & ((1 << E2M1_MAN_BITS) - 1)
    frac = m / (1 << E2M1_MAN_BITS)
    if e == 0:
        return sign * frac * 2.0 ** (1 - E2M1_BIAS)
    return sign * (1.0 + frac) * 2.0 ** (e - E2M1_BIAS)


def fp4_levels_f32() -> np.ndarray:
    """FP4 as a 16-entry table (a reading: the pages name FP4 -- irregular6612
    "QLoRA - Efficient Finetuning of Quantized LLMs" and itwiki "QLoRA" compare
    NF4 with it -- but give no grid): the values of all 16 bit patterns of the
    4-bit float E2M1, sorted ascending and divided by the largest magnitude so
    that they span [-1, 1].  Its two zeros (+0 and -0) sit at codes 7 and 8;
    both are stored as +0 (reading: a code that means zero dequantizes to +0)."""
    vals = np.array([e2m1_value(b) for b in range(16)], dtype=F64)
    vals = np.sort(vals) / np.max(np.abs(vals))
    vals[vals == 0.0] = 0.0                  # -0 -> +0
    return f32(vals)


# ---------------------------------------------------------------------------
# Blockwise quantization (itwiki "QLoRA", NF4 section; minnong511
# "quantization", block-wise quantization)
# ---------------------------------------------------------------------------

def blockwise_absmax(W: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """max |w| over consecutive runs of ``block`` elements of row-major W (fp32, exact)."""
    W = np.asarray(W, dtype=F32)
    return np.abs(W.reshape(-1, block)).max(axis=1)


def _nearest_level(x32: np.ndarray, levels32: np.ndarray) -> np.ndarray:
    """argmin_i |x - L_i| for an ascending level table, lowest index on an exact tie.

    x and L are fp32 values; each distance |x - L| is taken in fp64, rounded
    once, so it is within 2^-53 (relative) of the exact one.  Where the two
    nearest distinct levels are that close to equidistant -- an exact midpoint,
    or a tiny x between two levels of opposite sign -- the choice is made again
    in exact rational arithmetic.  Equal levels (FP4's two zeros) count once,
    under their lowest index.
    """
    L = np.asarray(levels32, dtype=F32).astype(F64)
    assert np.all(np.diff(L) >= 0), "levels must be ascending"
    uniq, first = np.unique(L, return_index=True)
    x = np.asarray(x32, dtype=F32)
    d = np.abs(x.astype(F64)[..., None] - uniq)
    k = np.argmin(d, axis=-1)
    two = np.partition(d, 1, axis=-1)
    unsure = two[..., 1] - two[..., 0] <= 2.0 ** -50 * two[..., 1]
    if np.any(unsure):
        Lq = [Fraction(float(v)) for v in uniq]
        for pos in zip(*np.nonzero(unsure)):
            xv = Fraction(float(x[pos]))
            k[pos] = min(range(len(Lq)), key=lambda i: (abs(xv - Lq[i]), i))
    return first[k].astype(np.uint8)


def quantize_codes(W: np.ndarray, levels32: np.ndarray | None = None,
                   block: int = BLOCK, chunk_blocks: int = 8192):
    """Quantize row-major fp32 W blockwise.  Returns (codes u8 [W.size], absmax fp32).

    Each block is divided by its absmax (one IEEE fp32 division per element)
    and every quotient is mapped to its nearest level.  A block whose absmax is
    0 gets, for every element, the level nearest to 0 (code 7 for NF4).
    """
    L = nf4_levels_f32() if levels32 is None else np.asarray(levels32, dtype=F32)
    W = np.asarray(W, dtype=F32).reshape(-1, block)
    absmax = np.abs(W).max(axis=1)
    zero_code = np.uint8(np.argmin(np.abs(L.astype(F64))))
    codes = np.empty(W.shape, dtype=np.uint8)
    for b0 in range(0, W.shape[0], chunk_blocks):
        w = W[b0:b0 + chunk_blocks].astype(F64)
        a = absmax[b0:b0 + chunk_blocks].astype(F64)
        nz = a > 0
        x = np.zeros_like(w)
        x[nz] = w[nz] / a[nz, None]
        c = _nearest_level(f32(x), L)
        c[~nz] = zero_code
        codes[b0:b0 + chunk_blocks] = c
    return codes.reshape(-1), absmax


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element 2i in the low nibble, 2i+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out


def nf4_quantize(W: np.ndarray, levels32: np.ndarray | None = None):
    """W fp32 [N, K] (K % 64 == 0) -> packed codes u8 [N, K/2], absmax fp32 [N*K/64]
    (NF4 levels unless another 16-level table is given)."""
    N, K = W.shape
    assert K % BLOCK == 0
    codes, absmax = quantize_codes(W, levels32)
    return pack_nibbles(codes).reshape(N, K // 2), absmax


# ---------------------------------------------------------------------------
# 8-bit float (OCP E4M3FN) from its definition
# ---------------------------------------------------------------------------

def e4m3_value(code) -> np.ndarray:
    """Decode E4M3FN bytes: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN; there is
    no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(F64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(F64)))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


_E4M3_MAGS = e4m3_value(np.arange(0x7F))   # codes 0x00..0x7E: 0 .. 448, increasing


def e4m3_encode(t32: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3FN byte: nearest finite value, ties to the even mantissa,
    magnitudes beyond 448 saturate to 448, and the sign is kept (also for 0)."""
    t = np.asarray(t32, dtype=F32).astype(F64)
    neg = np.signbit(t)
    a = np.minimum(np.abs(t), E4M3_MAX)
    hi = np.searchsorted(_E4M3_MAGS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_MAGS[lo]
    d_hi = _E4M3_MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    mag_code = np.where(pick_hi, hi, lo)
    mag_code = np.where(a == _E4M3_MAGS[hi], hi, mag_code)     # exact hits
    return (mag_code | (neg.astype(np.int64) << 7)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Double quantization (itwiki "QLoRA", double quantization section)
# ---------------------------------------------------------------------------

def round_rational_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32, ties to even (normal and subnormal)."""
    if q == 0:
        return F32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    k = q / ulp
    n = k.numerator // k.denominator
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = Fraction(n) * ulp
    return F32(sign * float(value))   # value is an fp32 number, so float() is exact


def exact_sum_f32(values: np.ndarray) -> Fraction:
    """The exact sum of fp32 values as a rational.

    Every finite fp32 v is an integer multiple of 2^-149: v * 2^149 = mant * 2^(e-1)
    with e the biased exponent (e >= 1, implicit bit set) or mant * 2^0 for
    subnormals.  Mantissas are summed per exponent in int64 and combined as
    Python integers, so nothing is rounded.
    """
    v = np.ascontiguousarray(values, dtype=F32).reshape(-1)
    bits = v.view(np.uint32)
    sign = (bits >> 31).astype(np.int64)
    e = ((bits >> 23) & 0xFF).astype(np.int64)
    mant = (bits & 0x7FFFFF).astype(np.int64)
    mant = np.where(e > 0, mant | 0x800000, mant)
    mant = np.where(sign == 1, -mant, mant)
    shift = np.maximum(e, 1) - 1
    total = 0
    for s in np.unique(shift):
        total += int(mant[shift == s].sum(dtype=np.int64)) << int(s)
    return Fraction(total, 1 << 149)


def mean_f32(values: np.ndarray) -> np.float32:
    """The arithmetic mean of fp32 values, exact, rounded once to fp32."""
    v = np.asarray(values, dtype=F32).reshape(-1)
    return round_rational_to_f32(exact_sum_f32(v) / v.size)


def double_quant(absmax: np.ndarray):
    """absmax fp32 [n] -> (c2 u8 [n], c1 fp32 [ceil(n/256)], mu fp32).

    The constants are all positive, so the tensor mean mu is subtracted first;
    each run of 256 centred constants is then scaled so that its largest
    magnitude maps to the largest E4M3 value (c1 = amax / 448, one fp32 per
    run) and rounded to E4M3.  A run whose scale is 0 stores code 0.
    """
    a = np.asarray(absmax, dtype=F32).reshape(-1)
    n = a.size
    mu = mean_f32(a)
    x = f32(a.astype(F64) - F64(mu))
    nb = -(-n // DQ_BLOCK)
    xp = np.zeros(nb * DQ_BLOCK, dtype=F32)
    xp[:n] = x
    xp = xp.reshape(nb, DQ_BLOCK)
    amax = np.abs(xp).max(axis=1)
    c1 = f32(amax.astype(F64) / E4M3_MAX)
    t = np.zeros_like(xp)
    ok = c1 > 0
    t[ok] = f32(xp[ok].astype(F64) / c1[ok, None].astype(F64))
    c2 = e4m3_encode(t).reshape(-1)[:n]
    c2[np.repeat(~ok, DQ_BLOCK)[:n]] = 0
    return c2, c1, mu


def dequant_constants(c2: np.ndarray, c1: np.ndarray, mu) -> np.ndarray:
    """c_hat = fp32( fp32(e4m3(c2) * c1) + mu ): two separate roundings, no fused multiply-add."""
    c2 = np.asarray(c2, dtype=np.uint8).reshape(-1)
    idx = np.arange(c2.size) // DQ_BLOCK
    prod = f32(e4m3_value(c2) * np.asarray(c1, dtype=F32)[idx].astype(F64))
    return f32(prod.astype(F64) + F64(F32(mu)))


# ---------------------------------------------------------------------------
# bf16 and weight dequantization (itwiki "QLoRA", computation section)
# ---------------------------------------------------------------------------

def bf16_round(v32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (8 significant bits, ties to even); returns the bf16 bits."""
    v = np.asarray(v32, dtype=F32).astype(F64)
    _, e = np.frexp(v)                          # v = m * 2^e with 0.5 <= |m| < 1
    ulp_exp = np.maximum(e, -125) - 8           # bf16 spacing; fixed 2^-133 below 2^-126
    q = np.rint(np.ldexp(v, -ulp_exp))          # rint rounds half to even
    r = np.ldexp(q, ulp_exp)
    return (f32(r).view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(F32).astype(F64)


def dequant_weight(codes_packed: np.ndarray, c2: np.ndarray, c1: np.ndarray, mu,
                   N: int, K: int, rows=None, levels32: np.ndarray | None = None) -> np.ndarray:
    """W_deq = bf16( fp32( L[code] * c_hat ) ) as bf16 bits [len(rows), K].

    ``rows`` selects output rows (default all); codes and constants are given
    for the whole tensor.
    """
    L = nf4_levels_f32() if levels32 is None else np.asarray(levels32, dtype=F32)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    packed = np.asarray(codes_packed, dtype=np.uint8).reshape(N, K // 2)[rows]
    codes = unpack_nibbles(packed).reshape(len(rows), K)
    nblk = K // BLOCK
    blk = rows[:, None] * nblk + np.arange(nblk)[None, :]          # [rows, K/64]
    c2r = np.asarray(c2, dtype=np.uint8)[blk]
    c1r = np.asarray(c1, dtype=F32)[blk // DQ_BLOCK]
    prod = f32(e4m3_value(c2r) * c1r.astype(F64))
    chat = f32(prod.astype(F64) + F64(F32(mu)))                     # [rows, K/64]
    return dequant_codes(codes, chat, L)


def dequant_codes(codes: np.ndarray, chat: np.ndarray, levels32: np.ndarray | None = None) -> np.ndarray:
    """W_deq = bf16( fp32( L[code] * c_hat ) ) for unpacked codes [R, nb*64] whose
    64-element blocks have the dequantized constants chat [R, nb]; bf16 bits [R, nb*64].

    Any set of whole blocks can be expanded this way (rows of W, or a 64-column
    slice of every row), since each block carries its own constant.
    """
    L = nf4_levels_f32() if levels32 is None else np.asarray(levels32, dtype=F32)
    codes = np.asarray(codes, dtype=np.uint8)
    R, n = codes.shape
    chat_e = np.repeat(np.asarray(chat, dtype=F32).reshape(R, n // BLOCK), BLOCK, axis=1)
    w = f32(L[codes].astype(F64) * chat_e.astype(F64))
    return bf16_round(w)


# ---------------------------------------------------------------------------
# The layer (itwiki "QLoRA" computation section; minnong511 "quantization")
# ---------------------------------------------------------------------------

def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / r, the LoRA branch scale, formed as one fp32 division."""
    return float(F32(F64(F32(alpha)) / F64(F32(r))))


def linear_fwd_f64(X, W, A, B, s: float):
    """Y = X W^T + s (X A^T) B^T on fp64 arrays; X [M,K], W [N,K], A [r,K], B [N,r]."""
    H = X @ A.T
    return X @ W.T + s * (H @ B.T), H


def linear_bwd_f64(dY, X, W, A, B, s: float) -> dict:
    """Gradients of <dY, Y> for X, A and B (W is frozen, so it gets none).

    With H = X A^T:  dH = s dY B,  dB = s dY^T H,  dA = dH^T X,  dX = dY W + dH A.
    """
    H = X @ A.T
    dH = s * (dY @ B)
    return {"dX": dY @ W + dH @ A, "dA": dH.T @ X, "dB": s * (dY.T @ H), "dH": dH, "H": H}


def linear_fwd(X_bits, Wdeq_bits, A_bits, B_bits, alpha: float, r: int):
    """The layer forward from bf16 operands (bits).  Returns (Y, H) in fp64."""
    return linear_fwd_f64(bf16_to_f64(X_bits), bf16_to_f64(Wdeq_bits), bf16_to_f64(A_bits),
                          bf16_to_f64(B_bits), lora_scale(alpha, r))


def linear_bwd(dY_bits, X_bits, Wdeq_bits, A_bits, B_bits, alpha: float, r: int) -> dict:
    """The layer backward from bf16 operands (bits): dX, dA, dB (and dH, H) in fp64."""
    return linear_bwd_f64(bf16_to_f64(dY_bits), bf16_to_f64(X_bits), bf16_to_f64(Wdeq_bits),
                          bf16_to_f64(A_bits), bf16_to_f64(B_bits), lora_scale(alpha, r))


def storage_bits_per_param(N: int, K: int) -> float:
    """Bits per parameter of the stored constants (c2 bytes, c1 floats, the mean)."""
    n_c2 = N * K // BLOCK
    n_c1 = -(-n_c2 // DQ_BLOCK)
    return (8 * n_c2 + 32 * n_c1 + 32) / (N * K)


def quantize_layer(W: np.ndarray, levels32: np.ndarray | None = None):
    """Full quantization of one fp32 weight: packed codes, absmax, c2, c1, mu
    (NF4 levels unless another 16-level table is given)."""
    codes, absmax = nf4_quantize(W, levels32)
    c2, c1, mu = double_quant(absmax)
    return {"codes": codes, "absmax": absmax, "c2": c2, "c1": c1, "mu": mu}


def bf16_round_f64(v64: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 in one step (8 significant bits, ties to even,
    bf16 subnormals below 2^-126); returns the bf16 bits.  Finite inputs below
    2^128 in magnitude."""
    v = np.asarray(v64, dtype=F64)
    _, e = np.frexp(v)
    ulp_exp = np.maximum(e, -125) - 8
    q = np.rint(np.ldexp(v, -ulp_exp))          # exact scaling; rint rounds half to even
    r = np.ldexp(q, ulp_exp)                    # 8 significant bits: exact in fp32
    return (f32(r).view(np.uint32) >> 16).astype(np.uint16)


def merge_weight(Wdeq_bits, A_bits, B_bits, alpha: float, r: int) -> np.ndarray:
    """The merged weight W_deq + s B A as bf16 bits [N, K] (irregular6612 "QLoRA -
    Efficient Finetuning of Quantized LLMs": after training the adapter is
    folded into the dequantized bf16 base weight; minnong511 "quantization":
    W' = W + (alpha / r) B A).

    Arithmetic, in fp64: the product B A summed over j in ascending order (each
    product of two bf16 numbers is exact; one rounding per addition), that sum
    times s (one rounding), plus W_deq (one rounding), then one rounding to
    bf16."""
    s = F64(lora_scale(alpha, r))
    A = bf16_to_f64(A_bits).reshape(r, -1)
    B = bf16_to_f64(B_bits).reshape(-1, r)
    W = bf16_to_f64(Wdeq_bits).reshape(B.shape[0], A.shape[1])
    acc = np.zeros_like(W)
    for j in range(r):
        acc = acc + B[:, j:j + 1] * A[j:j + 1, :]
    return bf16_round_f64(W + s * acc)


def quantize_layer_bf16(W_bits: np.ndarray):
    """Quantization of a bf16 weight (uint16 bit patterns): minnong511
    "quantization", the QLoRA pipeline, quantizes the base model's FP16/BF16
    weights to 4 bits.  A bf16 number is an fp32 number with the low 16 bits
    zero, so it widens exactly and is then quantized as an fp32 weight."""
    bits = np.asarray(W_bits, dtype=np.uint16)
    W = (bits.astype(np.uint32) << 16).view(F32)
    return quantize_layer(W)
