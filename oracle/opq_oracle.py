"""Plain, slow CPU oracle for OPQ (Optimal Power Quantization): 4-bit codes
(and 3, 5 and 6-bit ones further down) with one scale per output row or one
float16 scale per group of weights.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code,
table or constant generator with the HIP library and imports nothing from it.

Source of every step: the model card "OPQ INT4 Z-Image: 最优幂次量化扩散模型推理"
(huggingpeers.co/models/dfytensor/OPQ-INT4-Z-Image):

* section "OPQ 原理" (OPQ principle): normalise u = |w| / max|w|, compand
  v = u^alpha, code q = round(15 v), reconstruct w' = sign(w) (q/15)^(1/alpha) max|w|;
* section "技术细节 / 存储格式" (storage format): a 4-bit magnitude, eight per
  uint32; a 1-bit sign plane, thirty-two per uint32; one max per group;
* section "技术细节 / 推理解码" (decode): q/15, raised to 1/alpha, times sign
  and the group max.

Readings taken where the page is silent:

* the max is taken per output row and kept as an fp32 scale (the card keeps an
  fp16 max per group of 128; the per-row form is the workload's);
* alpha is the exact binary32 value the caller passes;
* u is the IEEE binary32 quotient |w| / m rounded to nearest even, with
  subnormals kept; q is the integer nearest to 15 u^alpha evaluated exactly,
  halves going up (an exact half happens only for alpha = 1, u = 1/2);
* the sign bit is 1 exactly when w < 0 (so -0.0 gives 0), and a code of 0
  always reconstructs to +0.0;
* packing is little-endian along K: code k of a row sits in bits 4(k%8)..4(k%8)+3
  of word k//8, sign k in bit k%32 of word k//32;
* a row whose max is 0 gets scale 0, all codes 0 and all signs 0;
* the reconstruction is the real value sign (q/15)^(1/alpha) m rounded once to
  bfloat16 (round to nearest even); here it is evaluated in float64 first;
* the linear layer is y = x W'^T (+ bias) over the bf16 reconstructions,
  accumulated here in float64;
* the group-wise form (the card's own stored format) is described where it is
  defined, below.

Every function below is pinned by the CPU tests in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math

import mpmath
import numpy as np

LEVELS = 15          # 4-bit magnitude codes 0..15 ("q = round(v x 15)")
CODES_PER_WORD = 8   # "8 个打包进 1 个 uint32"
SIGNS_PER_WORD = 32  # "32 个打包进 1 个 uint32"

__all__ = [
    "LEVELS", "alpha_f32", "bf16_bits_to_f32", "f64_to_bf16_bits", "row_absmax",
    "encode", "pack", "unpack", "quantize", "reconstruct", "dequantize",
    "linear", "snr_db", "error_sums", "decision_thresholds_f32", "codes_of_u",
    "F16_MAX", "group_absmax_f16", "encode_grouped", "quantize_grouped",
    "reconstruct_grouped", "dequantize_grouped", "levels_of", "encode_bits", "pack_bits",
    "unpack_bits", "quantize_bits", "dequantize_bits", "error_sums_bits",
]


# ---------------------------------------------------------------- number formats

def alpha_f32(alpha: float) -> float:
    """The exact binary32 value of alpha, as a Python float."""
    return float(np.float32(alpha))


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32; exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f64_to_bf16_bits(d) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even) in one step.

    bfloat16 has 8 significant bits and binary32's exponent range; below
    2^-126 its spacing is the fixed 2^-133.  Values past the largest finite
    bfloat16 after rounding become infinity.  NaN is not expected here.
    """
    d = np.asarray(d, dtype=np.float64)
    neg = np.signbit(d)
    a = np.abs(d)
    _, e = np.frexp(a)                       # a = f * 2^e with f in [0.5, 1)
    quantum_exp = np.maximum(e.astype(np.int64) - 8, -133)
    k = np.rint(np.ldexp(a, -quantum_exp))   # exact scaling, ties to even
    val = np.ldexp(k, quantum_exp)           # representable in bfloat16 (or 2^128)
    with np.errstate(over="ignore"):
        f32 = val.astype(np.float32)         # exact, or inf past the range
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(neg, bits | np.uint16(0x8000), bits).astype(np.uint16)


# ---------------------------------------------------------------- quantizer

def row_absmax(w32: np.ndarray) -> np.ndarray:
    """m_n = max_k |w[n,k]| in float32 ("max(|w|)"); exact in any order."""
    w32 = np.asarray(w32, dtype=np.float32)
    if w32.shape[1] == 0:
        return np.zeros(w32.shape[0], np.float32)
    return np.max(np.abs(w32), axis=1).astype(np.float32)


def _nearest_code_exact(u: float, alpha: float, levels: int = LEVELS) -> int:
    """round(levels u^alpha) at 200 bits; halves go up."""
    with mpmath.workprec(200):
        v = mpmath.mpf(levels) * mpmath.power(mpmath.mpf(u), mpmath.mpf(alpha))
        fl = mpmath.floor(v)
        q = int(fl) + (1 if v - fl >= mpmath.mpf(0.5) else 0)
    return min(max(q, 0), levels)


def encode(w32: np.ndarray, alpha: float):
    """Codes, signs and scales of a float32 matrix w[N, K].

    Steps of the card's "OPQ 原理": u = |w| / max|w| (binary32 division),
    v = u^alpha, q = round(15 v).  Returns (q uint8 [N,K], s uint8 [N,K],
    scale float32 [N]).
    """
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    m = row_absmax(w32)
    absw = np.abs(w32)
    u = np.zeros_like(absw)
    live = m > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        u[live] = absw[live] / m[live, None]          # IEEE binary32 quotient
    q = codes_of_u(u, alpha)
    s = (w32 < 0).astype(np.uint8)                    # -0.0 is not < 0
    return q, s, m


def codes_of_u(u: np.ndarray, alpha: float, levels: int = LEVELS) -> np.ndarray:
    """q = round(levels u^alpha) for binary32 u >= 0, halves up, limited to
    `levels` (u above 1 only arises against a rounded group max)."""
    a64 = alpha_f32(alpha)
    v = levels * np.power(u.astype(np.float64), a64)
    q = np.floor(v + 0.5)
    # Values whose float64 v sits next to a half are settled exactly.
    frac = v - np.floor(v)
    for r, c in np.argwhere(np.abs(frac - 0.5) < 1e-9):
        q[r, c] = _nearest_code_exact(float(u[r, c]), a64, levels)
    return np.clip(q, 0, levels).astype(np.uint8)


def pack(q: np.ndarray, s: np.ndarray):
    """Pack codes eight per uint32 and signs thirty-two per uint32 (K order,
    least significant first).  K must be a multiple of 32."""
    q = np.asarray(q, dtype=np.uint32)
    s = np.asarray(s, dtype=np.uint32)
    n, k = q.shape
    assert k % SIGNS_PER_WORD == 0
    qg = q.reshape(n, k // CODES_PER_WORD, CODES_PER_WORD)
    packed = np.zeros((n, k // CODES_PER_WORD), np.uint32)
    for i in range(CODES_PER_WORD):
        packed |= (qg[:, :, i] & np.uint32(0xF)) << np.uint32(4 * i)
    sg = s.reshape(n, k // SIGNS_PER_WORD, SIGNS_PER_WORD)
    sign = np.zeros((n, k // SIGNS_PER_WORD), np.uint32)
    for i in range(SIGNS_PER_WORD):
        sign |= (sg[:, :, i] & np.uint32(1)) << np.uint32(i)
    return packed, sign


def unpack(packed: np.ndarray, sign: np.ndarray):
    """Inverse of :func:`pack`: (q uint8 [N,K], s uint8 [N,K])."""
    packed = np.asarray(packed, dtype=np.uint32)
    sign = np.asarray(sign, dtype=np.uint32)
    n, kw = packed.shape
    q = np.zeros((n, kw, CODES_PER_WORD), np.uint8)
    for i in range(CODES_PER_WORD):
        q[:, :, i] = (packed >> np.uint32(4 * i)) & np.uint32(0xF)
    s = np.zeros((n, sign.shape[1], SIGNS_PER_WORD), np.uint8)
    for i in range(SIGNS_PER_WORD):
        s[:, :, i] = (sign >> np.uint32(i)) & np.uint32(1)
    return q.reshape(n, -1), s.reshape(n, -1)


def quantize(w32: np.ndarray, alpha: float):
    """Quantize w[N, K] (float32 values) to (packed, sign, scale)."""
    q, s, m = encode(w32, alpha)
    packed, sign = pack(q, s)
    return packed, sign, m


# ---------------------------------------------------------------- dequantizer

def reconstruct(q: np.ndarray, s: np.ndarray, scale: np.ndarray, alpha: float,
                levels: int = LEVELS) -> np.ndarray:
    """w' = sign (q/15)^(1/alpha) m in float64 (section "推理解码"); q = 0 gives +0.
    `levels` replaces 15 for other code widths."""
    a64 = alpha_f32(alpha)
    q64 = np.asarray(q, dtype=np.float64)
    mag = np.power(q64 / levels, 1.0 / a64) * np.asarray(scale, np.float64)[:, None]
    neg = (np.asarray(s) != 0) & (np.asarray(q) != 0)
    return np.where(neg, -mag, mag)


def dequantize(packed: np.ndarray, sign: np.ndarray, scale: np.ndarray, alpha: float) -> np.ndarray:
    """Dequantize to bfloat16 bit patterns (uint16 [N, K]), rounded once."""
    q, s = unpack(packed, sign)
    return f64_to_bf16_bits(reconstruct(q, s, scale, alpha))


# ---------------------------------------------------------------- group-wise scales
#
# The card's stored form ("技术细节 / 存储格式"): one float16 max per group of
# weights ("每 128 个权重共享一个"; the configuration section offers group
# sizes 32, 64, 128 and 256), and the decode multiplies by that group max
# ("推理解码").  Readings: a group is `gs` consecutive weights of a row along K;
# the stored max is max|w| over the group rounded to float16 (nearest, ties to
# even; values past 65504 saturate to 65504); u is the binary32 quotient by the
# stored max, so u may exceed 1 by less than 2^-11 and then codes 15; a group
# whose stored max is 0 has all codes 0.

F16_MAX = 65504.0


def group_absmax_f16(w32: np.ndarray, gs: int) -> np.ndarray:
    """Stored group maxima, float16 [N, K/gs]."""
    w32 = np.asarray(w32, dtype=np.float32)
    n, k = w32.shape
    assert k % gs == 0
    if k == 0:
        return np.zeros((n, 0), np.float16)
    a = np.max(np.abs(w32).reshape(n, k // gs, gs), axis=2)
    return np.minimum(a, np.float32(F16_MAX)).astype(np.float16)   # numpy: nearest even


def encode_grouped(w32: np.ndarray, alpha: float, gs: int):
    """(q uint8 [N,K], s uint8 [N,K], m16 float16 [N,K/gs]) of w[N, K]."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    m16 = group_absmax_f16(w32, gs)
    m = np.repeat(m16.astype(np.float32), gs, axis=1)   # each weight's stored max
    absw = np.abs(w32)
    u = np.zeros_like(absw)
    live = m > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        u[live] = absw[live] / m[live]                 # IEEE binary32 quotient
    q = codes_of_u(u, alpha)
    s = (w32 < 0).astype(np.uint8)
    return q, s, m16


def quantize_grouped(w32: np.ndarray, alpha: float, gs: int):
    """(packed, sign, m16) of w[N, K] with one float16 max per gs weights."""
    q, s, m16 = encode_grouped(w32, alpha, gs)
    packed, sign = pack(q, s)
    return packed, sign, m16


def reconstruct_grouped(q, s, m16, alpha: float, gs: int) -> np.ndarray:
    """w' = sign (q/15)^(1/alpha) m16 in float64; q = 0 gives +0."""
    scale = np.repeat(np.asarray(m16, np.float16).astype(np.float64), gs, axis=1)
    a64 = alpha_f32(alpha)
    mag = np.power(np.asarray(q, np.float64) / LEVELS, 1.0 / a64) * scale
    neg = (np.asarray(s) != 0) & (np.asarray(q) != 0)
    return np.where(neg, -mag, mag)


def dequantize_grouped(packed, sign, m16, alpha: float, gs: int) -> np.ndarray:
    """bfloat16 bit patterns (uint16 [N, K]) of the group-wise stored form."""
    q, s = unpack(packed, sign)
    return f64_to_bf16_bits(reconstruct_grouped(q, s, m16, alpha, gs))


# ---------------------------------------------------------------- other code widths
#
# The card's configuration offers 3, 4, 5 or 6 bits ("OPQ_BITS"); its formulas
# are written for 4 (x 15, 16 levels).  Reading: b bits give 2^b - 1 in place
# of 15 everywhere (q = round((2^b - 1) u^alpha), w' = (q / (2^b - 1))^(1/alpha)
# m); the sign plane and the per-row max are unchanged.  The card gives no
# packing for b != 4; here the codes of a row form a little-endian bit stream
# along K, code k in bits b k .. b k + b - 1, so 32 codes fill b uint32 words
# (for b = 4 that is the nibble packing above).

def levels_of(bits: int) -> int:
    """Largest code of a b-bit magnitude: 2^b - 1 (15 for 4 bits)."""
    assert bits in (3, 4, 5, 6)
    return (1 << bits) - 1


def encode_bits(w32: np.ndarray, alpha: float, bits: int):
    """(q uint8 [N,K], s uint8 [N,K], scale float32 [N]) with b-bit codes."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    m = row_absmax(w32)
    absw = np.abs(w32)
    u = np.zeros_like(absw)
    live = m > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        u[live] = absw[live] / m[live, None]          # IEEE binary32 quotient
    q = codes_of_u(u, alpha, levels_of(bits))
    s = (w32 < 0).astype(np.uint8)
    return q, s, m


def pack_bits(q: np.ndarray, bits: int) -> np.ndarray:
    """Codes [N, K] as a bit stream per row: uint32 [N, K*bits/32]."""
    q = np.asarray(q, dtype=np.uint64)
    n, k = q.shape
    assert k % 32 == 0
    out = np.zeros((n, k * bits // 32), np.uint64)
    for i in range(k):
        pos = bits * i
        w, off = pos // 32, pos % 32
        out[:, w] |= (q[:, i] << np.uint64(off)) & np.uint64(0xFFFFFFFF)
        if off + bits > 32:
            out[:, w + 1] |= q[:, i] >> np.uint64(32 - off)
    return out.astype(np.uint32)


def unpack_bits(packed: np.ndarray, bits: int, k: int) -> np.ndarray:
    """Inverse of :func:`pack_bits`: codes uint8 [N, K]."""
    p = np.asarray(packed, dtype=np.uint64)
    n = p.shape[0]
    q = np.zeros((n, k), np.uint8)
    mask = np.uint64((1 << bits) - 1)
    for i in range(k):
        pos = bits * i
        w, off = pos // 32, pos % 32
        v = p[:, w] >> np.uint64(off)
        if off + bits > 32:
            v |= p[:, w + 1] << np.uint64(32 - off)
        q[:, i] = (v & mask).astype(np.uint8)
    return q


def quantize_bits(w32: np.ndarray, alpha: float, bits: int):
    """(packed [N, K*bits/32], sign [N, K/32], scale [N]) with b-bit codes."""
    q, s, m = encode_bits(w32, alpha, bits)
    _, sign = pack(np.zeros_like(q), s)
    return pack_bits(q, bits), sign, m


def dequantize_bits(packed, sign, scale, alpha: float, bits: int) -> np.ndarray:
    """bfloat16 bit patterns [N, K] of the b-bit stored form, rounded once."""
    k = np.asarray(sign).shape[1] * SIGNS_PER_WORD
    q = unpack_bits(packed, bits, k)
    _, s = unpack(np.zeros((q.shape[0], k // CODES_PER_WORD), np.uint32), sign)
    return f64_to_bf16_bits(reconstruct(q, s, scale, alpha, levels_of(bits)))


def error_sums_bits(w32: np.ndarray, alpha: float, bits: int) -> np.ndarray:
    """Per row: (sum w^2, sum (w - w')^2) in float64 for b-bit codes."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    packed, sign, scale = quantize_bits(w32, alpha, bits)
    w_rec = bf16_bits_to_f32(dequantize_bits(packed, sign, scale, alpha, bits)).astype(np.float64)
    w64 = w32.astype(np.float64)
    e = w64 - w_rec
    return np.stack([np.sum(w64 * w64, axis=1), np.sum(e * e, axis=1)], axis=1)


# ---------------------------------------------------------------- linear layer

def linear(x_bf16: np.ndarray, wdq_bf16: np.ndarray, bias=None) -> np.ndarray:
    """y[M, N] = x[M, K] . W'[N, K]^T (+ bias[N]) over bf16 inputs, in float64.

    x and W' are bfloat16 bit patterns; every product is exact in float64.
    """
    x = bf16_bits_to_f32(x_bf16).astype(np.float64)
    w = bf16_bits_to_f32(wdq_bf16).astype(np.float64)
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def error_sums(w32: np.ndarray, alpha: float) -> np.ndarray:
    """Per row of w[N, K]: (sum w^2, sum (w - w')^2) in float64, w' the bfloat16
    reconstruction of w's stored form (quantize then dequantize).  The card's
    section "为什么 α=0.73？" picks alpha from the flat optimum of this error;
    "OPQ 原理" compares it against uniform rounding (alpha = 1)."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    packed, sign, scale = quantize(w32, alpha)
    w_rec = bf16_bits_to_f32(dequantize(packed, sign, scale, alpha)).astype(np.float64)
    w64 = w32.astype(np.float64)
    e = w64 - w_rec
    return np.stack([np.sum(w64 * w64, axis=1), np.sum(e * e, axis=1)], axis=1)


def snr_db(w: np.ndarray, w_rec: np.ndarray) -> float:
    """10 log10(sum w^2 / sum (w - w')^2) over a whole tensor, in float64."""
    w = np.asarray(w, np.float64)
    e = w - np.asarray(w_rec, np.float64)
    num = float(np.sum(w * w))
    den = float(np.sum(e * e))
    if den == 0.0:
        return math.inf
    return 10.0 * math.log10(num / den)


# ---------------------------------------------------------------- decision points

def decision_thresholds_f32(alpha: float, levels: int = LEVELS) -> np.ndarray:
    """T_k = the smallest binary32 t with 15 t^alpha >= k - 1/2, k = 1..15
    (`levels` in place of 15 for other code widths).

    For binary32 u in [0, 1], round(15 u^alpha) (halves up) equals the number
    of k with u >= T_k.  Computed with mpmath at 200 bits: the real boundary
    ((2k-1)/30)^(1/alpha) is rounded to binary32 and stepped up or down by one
    ulp until the condition holds at T_k and fails one ulp below.
    """
    a = alpha_f32(alpha)
    out = np.zeros(levels, np.float32)
    with mpmath.workprec(200):
        A = mpmath.mpf(a)

        def ok(t: np.float32, k: int) -> bool:
            v = levels * mpmath.power(mpmath.mpf(float(t)), A)
            return v >= k - mpmath.mpf(0.5)

        for k in range(1, levels + 1):
            b = mpmath.power(mpmath.mpf(2 * k - 1) / (2 * levels), 1 / A)
            t = np.float32(float(b))
            while not ok(t, k):
                t = np.nextafter(t, np.float32(np.inf))
            while t > 0 and ok(np.nextafter(t, np.float32(0)), k):
                t = np.nextafter(t, np.float32(0))
            out[k - 1] = t
    return out
