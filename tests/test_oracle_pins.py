"""Pins for the CPU oracle: closed forms, exact rational special cases,
brute force and invariants, each independent of the oracle's own code path.

The method is the model card "OPQ INT4 Z-Image" (section "OPQ 原理" for the
quantizer, "技术细节 / 存储格式" for packing, "技术细节 / 推理解码" for the
decode).  The card prints no worked numeric example, so the fixtures here are
closed forms and hand-built words (tests/golden/packing_example.txt).
"""
import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle as O
from tests.exact import bf16_bits_of, exact_quotient_f32, f32_of, round_fraction

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_rows(seed, n, k, scale=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_t(4, size=(n, k)) * scale).astype(np.float32)


def _to_bf16_values(w32):
    """Round float32 to bf16 with torch's cast, back to float32 values."""
    t = torch.from_numpy(np.ascontiguousarray(w32)).to(torch.bfloat16).to(torch.float32)
    return t.numpy()


# ------------------------------------------------------------------ number formats

def test_f64_to_bf16_agrees_with_torch_cast():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -2.0, 3.3895314e38, 1e-45, -1e-45], np.float32),
    ])
    # exact midpoints between neighbouring bf16 values: ties to even
    base = rng.integers(0x0080, 0x7F00, 4000).astype(np.uint32) << 16
    mids = (base | 0x8000).view(np.float32)
    vals = np.concatenate([vals, mids, -mids])
    mine = O.f64_to_bf16_bits(vals.astype(np.float64))
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_f64_to_bf16_exact_rational():
    """Float64 inputs that no float32 holds: compare with exact rounding."""
    rng = np.random.default_rng(12)
    d = rng.standard_normal(3000) * np.exp2(rng.integers(-130, 100, 3000))
    mine = O.f64_to_bf16_bits(d)
    ref = np.array([bf16_bits_of(Fraction(float(x))) for x in d], np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_widen_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x0000, 0x8000], np.uint16)
    v = O.bf16_bits_to_f32(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133
    assert np.isinf(v[3]) and v[4] == 0.0 and np.signbit(v[5])


# ------------------------------------------------------------------ absmax

def test_absmax_planted():
    w = _rand_rows(1, 17, 96)
    planted = np.float32(-0.731)
    w[5, 40] = planted
    m = O.row_absmax(w)
    assert m[5] == np.float32(0.731)
    assert np.all(m >= np.abs(w).max(axis=1)) and np.all(m <= np.abs(w).max(axis=1))


# ------------------------------------------------------------------ codes: exact closed forms

def _exact_u(w, m):
    return [[exact_quotient_f32(np.float32(abs(x)), np.float32(mm)) for x in row]
            for row, mm in zip(w, m)]


def _codes_closed_form(w, rule):
    m = np.max(np.abs(w), axis=1)
    us = _exact_u(w, m)
    return np.array([[rule(u) for u in row] for row in us], np.uint8)


def test_alpha_one_is_uniform_absmax_rounding():
    """alpha = 1: q = rint(15 u), the textbook symmetric absmax quantizer
    (the card's "传统均匀量化" baseline)."""
    w = _rand_rows(2, 6, 64)
    w[0, 3] = np.float32(0.5) * np.abs(w[0]).max()      # exact tie u = 1/2 -> 8
    q, _, _ = O.encode(w, 1.0)
    ref = _codes_closed_form(w, lambda u: int(np.rint(15 * float(u))))
    assert np.array_equal(q, ref)
    assert q[0, 3] == 8


@pytest.mark.parametrize("alpha,rule", [
    # 15 sqrt(u) >= k - 1/2  <=>  900 u >= (2k-1)^2
    (0.5, lambda u: sum(1 for k in range(1, 16) if 900 * u >= (2 * k - 1) ** 2)),
    # 15 u^2 >= k - 1/2      <=>  30 u^2 >= 2k-1
    (2.0, lambda u: sum(1 for k in range(1, 16) if 30 * u * u >= 2 * k - 1)),
    # 15 u^(1/4) >= k - 1/2  <=>  30^4 u >= (2k-1)^4
    (0.25, lambda u: sum(1 for k in range(1, 16) if 810000 * u >= (2 * k - 1) ** 4)),
])
def test_dyadic_alpha_exact_rational_codes(alpha, rule):
    w = _rand_rows(3, 6, 64)
    q, _, _ = O.encode(w, alpha)
    assert np.array_equal(q, _codes_closed_form(w, rule))


def test_special_values():
    w = _rand_rows(4, 4, 64)
    w[1, :] = 0.0
    w[1, 7] = -0.0
    w[2, 9] = -np.abs(w[2]).max() * 2          # the row max, negative
    w[3, 0] = -0.0
    w[3, 1] = np.float32(-1e-30)               # tiny negative: q = 0 but sign 1
    q, s, m = O.encode(w, 0.73)
    assert m[1] == 0 and not q[1].any() and not s[1].any()
    assert q[2, 9] == 15 and s[2, 9] == 1
    at_max = (np.abs(w) == m[:, None]) & (m[:, None] > 0)
    assert at_max.sum() >= 3 and np.all(q[at_max] == 15)
    assert q[3, 0] == 0 and s[3, 0] == 0
    assert q[3, 1] == 0 and s[3, 1] == 1
    assert np.all(q[w == 0] == 0)


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
def test_codes_monotone_in_magnitude(alpha):
    w = _rand_rows(5, 8, 512)
    q, _, _ = O.encode(w, alpha)
    for r in range(w.shape[0]):
        order = np.argsort(np.abs(w[r]), kind="stable")
        assert np.all(np.diff(q[r, order].astype(int)) >= 0)


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
def test_bruteforce_nearest_level(alpha):
    """Every code is the nearest of the 16 levels j in v-space,
    argmin_j |15 u^alpha - j| (ties to the larger j), in mpmath."""
    w = _rand_rows(6, 3, 32)
    q, _, m = O.encode(w, alpha)
    a = mpmath.mpf(O.alpha_f32(alpha))
    with mpmath.workprec(120):
        for r in range(w.shape[0]):
            for c in range(w.shape[1]):
                u = exact_quotient_f32(np.float32(abs(w[r, c])), m[r])
                v = 15 * mpmath.power(mpmath.mpf(u.numerator) / u.denominator, a)
                d = [abs(v - j) for j in range(16)]
                best = min(range(16), key=lambda j: (d[j], -j))
                assert q[r, c] == best, (r, c)


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
@pytest.mark.parametrize("m_bits", [0x3DCD, 0x3F80, 0x0100, 0x7F7F])
def test_exhaustive_bf16_sweep_against_inverse_boundaries(alpha, m_bits):
    """All non-negative bf16 a <= m: the code equals the count of real
    boundaries ((2k-1)/30)^(1/alpha) that u = fl32(a/m) reaches."""
    m = O.bf16_bits_to_f32(np.array([m_bits], np.uint16))[0]
    a_bits = np.arange(0, m_bits + 1, dtype=np.uint16)
    a = O.bf16_bits_to_f32(a_bits)
    w = a[None, :].astype(np.float32)
    q, _, mm = O.encode(w, alpha)
    assert mm[0] == m
    al = mpmath.mpf(O.alpha_f32(alpha))
    with mpmath.workprec(120):
        bounds = [mpmath.power(mpmath.mpf(2 * k - 1) / 30, 1 / al) for k in range(1, 16)]
    bf = np.array([float(b) for b in bounds])
    u32 = (a / m).astype(np.float32).astype(np.float64)
    ref = np.zeros(a.shape, np.int64)
    for k, b in enumerate(bf):
        near = np.abs(u32 - b) <= 1e-12 * b
        ref += (u32 >= b) & ~near
        for i in np.nonzero(near)[0]:
            uq = exact_quotient_f32(np.float32(a[i]), np.float32(m))
            with mpmath.workprec(120):
                ref[i] += int(mpmath.mpf(uq.numerator) / uq.denominator >= bounds[k])
    # the float32 quotient used for the bulk compare is the exact one
    for i in np.linspace(0, len(a) - 1, 97).astype(int):
        assert Fraction(float(u32[i])) == exact_quotient_f32(np.float32(a[i]), np.float32(m))
    assert np.array_equal(q[0].astype(np.int64), ref)


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
def test_fp32_near_threshold_sweep(alpha):
    """Inputs within +-40 ulps of each decision point in |w|-space: the code
    switches exactly where exact arithmetic on fl32(|w|/m) says."""
    m = np.float32(0.0371)
    al = mpmath.mpf(O.alpha_f32(alpha))
    vals = []
    for k in range(1, 16):
        with mpmath.workprec(120):
            b = mpmath.power(mpmath.mpf(2 * k - 1) / 30, 1 / al) * mpmath.mpf(float(m))
        c = np.float32(float(b))
        x = c
        for _ in range(40):
            x = np.nextafter(x, np.float32(0))
        for _ in range(81):
            if x <= m:
                vals.append(x)
            x = np.nextafter(x, np.float32(1))
    w = np.array([list(vals) + [m]], np.float32)
    q, _, mm = O.encode(w, alpha)
    assert mm[0] == m
    with mpmath.workprec(160):
        for i, x in enumerate(vals):
            u = exact_quotient_f32(x, m)
            uu = mpmath.mpf(u.numerator) / u.denominator
            ref = sum(1 for k in range(1, 16)
                      if 15 * mpmath.power(uu, al) >= k - mpmath.mpf(0.5))
            assert q[0, i] == ref, (k, i)


def test_decision_thresholds_rational_cases():
    """T_k for alpha = 1 and 1/2 are binary32 roundings up of rationals."""
    def up(fr):
        t = f32_of(fr)
        if Fraction(float(t)) < fr:
            t = np.nextafter(t, np.float32(2))
        return t
    t1 = O.decision_thresholds_f32(1.0)
    t_half = O.decision_thresholds_f32(0.5)
    for k in range(1, 16):
        assert t1[k - 1] == up(Fraction(2 * k - 1, 30))
        assert t_half[k - 1] == up(Fraction((2 * k - 1) ** 2, 900))
    assert t1[7] == np.float32(0.5)


@pytest.mark.parametrize("alpha", [0.3, 0.45, 0.73, 1.0, 2.0])
def test_decision_thresholds_are_least_in_class(alpha):
    """T_k is the least binary32 t with 15 t^alpha >= k - 1/2 ("OPQ 原理":
    code k from k - 1/2 up): T_k is in that class and the binary32 just below
    it is not, in 200-bit arithmetic."""
    al = mpmath.mpf(O.alpha_f32(alpha))
    t = O.decision_thresholds_f32(alpha)
    with mpmath.workprec(200):
        for k in range(1, 16):
            def in_class(x):
                return 15 * mpmath.power(mpmath.mpf(float(x)), al) >= k - mpmath.mpf(0.5)
            assert in_class(t[k - 1]), (alpha, k)
            assert not in_class(np.nextafter(t[k - 1], np.float32(0))), (alpha, k)


@pytest.mark.parametrize("alpha", [0.45, 0.73])
def test_encode_equals_threshold_count(alpha):
    w = _rand_rows(7, 16, 256)
    q, _, m = O.encode(w, alpha)
    u = (np.abs(w) / m[:, None]).astype(np.float32)
    t = O.decision_thresholds_f32(alpha)
    cnt = (u[:, :, None] >= t[None, None, :]).sum(axis=2)
    assert np.array_equal(q, cnt)


# ------------------------------------------------------------------ packing

def _golden_words():
    out = {}
    with open(os.path.join(GOLDEN, "packing_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                key, words = line.split(":")
                out[key.strip()] = [int(x, 16) for x in words.split()]
    return out


def test_packing_worked_example():
    g = _golden_words()
    k = np.arange(64)
    q = (k % 16).astype(np.uint8)[None, :]
    s = (k % 2).astype(np.uint8)[None, :]
    packed, sign = O.pack(q, s)
    assert list(packed[0]) == g["codes_k_mod_16"]
    assert list(sign[0]) == g["signs_odd_negative"]
    q2 = np.zeros((1, 64), np.uint8)
    q2[0, 37] = 0xB
    p2, _ = O.pack(q2, np.zeros_like(q2))
    assert list(p2[0]) == g["single_code_at_37"]


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(8)
    q = rng.integers(0, 16, (5, 96)).astype(np.uint8)
    s = rng.integers(0, 2, (5, 96)).astype(np.uint8)
    p, sg = O.pack(q, s)
    q2, s2 = O.unpack(p, sg)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("alpha,level", [
    (1.0, lambda q: Fraction(q, 15)),
    (0.5, lambda q: Fraction(q, 15) ** 2),
    (0.25, lambda q: Fraction(q, 15) ** 4),
])
def test_dequant_exact_rational(alpha, level):
    """For alpha = 1, 1/2, 1/4 the level (q/15)^(1/alpha) is rational: the
    bf16 reconstruction must be the exactly rounded value, bit for bit."""
    w = _to_bf16_values(_rand_rows(9, 8, 64))
    packed, sign, m = O.quantize(w, alpha)
    got = O.dequantize(packed, sign, m, alpha)
    q, s = O.unpack(packed, sign)
    for r in range(w.shape[0]):
        for c in range(w.shape[1]):
            v = level(int(q[r, c])) * Fraction(float(m[r]))
            if s[r, c] and q[r, c]:
                v = -v
            assert got[r, c] == bf16_bits_of(v), (r, c)


def test_dequant_rounds_once_near_midpoints():
    """Cases where the reconstruction lies just above a bf16 midpoint, within
    half a binary32 ulp: rounding through binary32 first would land on the
    midpoint and tie to even (down); rounding once goes up."""
    rng = np.random.default_rng(16)
    m = (1 + rng.random(1 << 20)).astype(np.float32)
    qs, ms = [], []
    for q in range(1, 15):
        v = q * m.astype(np.float64) / 15
        v32 = v.astype(np.float32)
        b = v32.view(np.uint32)
        hit = ((b & 0xFFFF) == 0x8000) & (v > v32) & (((b >> 16) & 1) == 0)
        qs += [q] * int(hit.sum())
        ms += list(m[hit])
    assert len(qs) >= 8
    n = len(qs)
    k = 32
    qq = np.zeros((n, k), np.uint8)
    qq[:, 0] = qs
    packed, sign = O.pack(qq, np.zeros_like(qq))
    scale = np.array(ms, np.float32)
    d = O.dequantize(packed, sign, scale, 1.0)
    for i in range(n):
        exact = Fraction(int(qs[i]), 15) * Fraction(float(scale[i]))
        assert d[i, 0] == bf16_bits_of(exact), i


def test_dequant_special_values():
    w = _to_bf16_values(_rand_rows(10, 4, 64))
    w[2, 5] = -0.0
    w[3, :] = 0
    packed, sign, m = O.quantize(w, 0.73)
    d = O.dequantize(packed, sign, m, 0.73)
    q, s = O.unpack(packed, sign)
    mbits = (m.view(np.uint32) >> 16).astype(np.uint16)
    for r in range(4):
        top = q[r] == 15
        assert np.all((d[r][top] & 0x7FFF) == mbits[r])      # max reconstructs exactly
    assert np.all(d[q == 0] == 0)                              # +0.0, never -0.0
    assert not d[3].any()


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
def test_quantize_dequantize_idempotent(alpha):
    w = _to_bf16_values(_rand_rows(11, 32, 512))
    p1, s1, m1 = O.quantize(w, alpha)
    d1 = O.dequantize(p1, s1, m1, alpha)
    w2 = O.bf16_bits_to_f32(d1)
    p2, s2, m2 = O.quantize(w2, alpha)
    d2 = O.dequantize(p2, s2, m2, alpha)
    assert np.array_equal(p1, p2)                  # codes unchanged
    assert np.array_equal(m1, m2)                  # the max is itself a level
    assert np.array_equal(d1, d2)


def test_reconstruction_error_bound():
    """|w - w'| <= half the gap to the neighbouring level plus a bf16 ulp
    (the quantizer is a nearest-level rule in v-space, so in w-space the
    error is bounded by the largest level gap)."""
    alpha = 0.73
    w = _to_bf16_values(_rand_rows(12, 8, 256))
    p, s, m = O.quantize(w, alpha)
    d = O.bf16_bits_to_f32(O.dequantize(p, s, m, alpha)).astype(np.float64)
    levels = (np.arange(16) / 15.0) ** (1 / O.alpha_f32(alpha))
    gap = np.max(np.diff(levels))
    err = np.abs(w.astype(np.float64) - d) / m[:, None]
    assert np.all(err <= gap + 2 ** -7)


# ------------------------------------------------------------------ linear

def test_linear_one_hot_rows_pick_columns():
    w = _to_bf16_values(_rand_rows(13, 24, 64))
    p, s, m = O.quantize(w, 0.73)
    wd = O.dequantize(p, s, m, 0.73)
    x = np.zeros((64, 64), np.float32)
    x[np.arange(64), np.arange(64)] = 1.0
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    y = O.linear(xb, wd)
    assert np.array_equal(y.T.astype(np.float32), O.bf16_bits_to_f32(wd))


def test_linear_exact_small():
    rng = np.random.default_rng(14)
    x = _to_bf16_values(rng.standard_normal((3, 32)).astype(np.float32))
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    w = _to_bf16_values(_rand_rows(15, 5, 32))
    p, s, m = O.quantize(w, 0.73)
    wd = O.dequantize(p, s, m, 0.73)
    wv = O.bf16_bits_to_f32(wd)
    bias = np.array([0.5, -1, 0, 2, 0.25], np.float32)
    y = O.linear(xb, wd, bias)
    for i in range(3):
        for j in range(5):
            ex = sum(Fraction(float(x[i, k])) * Fraction(float(wv[j, k])) for k in range(32))
            ex += Fraction(float(bias[j]))
            assert abs(Fraction(float(y[i, j])) - ex) <= Fraction(1, 2 ** 40)


# ------------------------------------------------------------------ SNR

def test_snr_closed_form():
    m = 0.8
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1] = m, m / 2                 # u = 1/2 exactly: q = round(7.5) = 8
    p, s, mm = O.quantize(w, 1.0)
    d = O.bf16_bits_to_f32(O.dequantize(p, s, mm, 1.0))
    mf = Fraction(float(np.float32(m)))
    assert d[0, 0] == float(round_fraction(mf, 8))
    assert d[0, 1] == float(round_fraction(Fraction(8, 15) * mf, 8))
    assert not d[0, 2:].any()
    assert O.snr_db(d, d) == math.inf


def test_snr_exact_cases():
    """Signal and error energies picked by hand so the ratio is a power of ten:
    w = (3, 4), w' = (3, 3.5): 25 / 0.25 = 100, 20 dB; w = (1, 3), w' = (0, 3):
    10 / 1, 10 dB; a tensor whose every error equals its own value: 0 dB.  A
    swapped ratio, an amplitude (not energy) ratio, a missing factor 10 or the
    error taken as w + w' each miss one of these."""
    assert O.snr_db(np.array([[3.0, 4.0]]), np.array([[3.0, 3.5]])) == 20.0
    assert O.snr_db(np.array([[1.0, 3.0]]), np.array([[0.0, 3.0]])) == 10.0
    assert O.snr_db(np.array([[1.0, 3.0], [0.0, 0.0]]), np.array([[0.0, 3.0], [0.0, 0.0]])) == 10.0
    assert O.snr_db(np.array([[0.5, -2.0]]), np.zeros((1, 2))) == 0.0


# ------------------------------------------------------------------ error sums (alpha sweep)

def _exact_code(u: Fraction, alpha_num: int) -> int:
    """round(15 u) for alpha = 1, halves up, in exact arithmetic."""
    v = 15 * u
    fl = v.numerator // v.denominator
    return fl + (1 if v - fl >= Fraction(1, 2) else 0)


def test_error_sums_closed_form_alpha1():
    """alpha = 1: codes are round(15 u) on the binary32 quotient and the
    reconstruction is bf16((q/15) m); the squared error is summed exactly."""
    m = np.float32(0.7)
    vals = [m, m / 2, np.float32(m / 3), -np.float32(m / 7), np.float32(0.05), -np.float32(0.31),
            np.float32(1e-3), np.float32(0.0)]
    w = np.zeros((1, 32), np.float32)
    w[0, :len(vals)] = vals
    got = O.error_sums(w, 1.0)
    mf = Fraction(float(m))
    sw2 = Fraction(0)
    se2 = Fraction(0)
    for a in w[0]:
        af = Fraction(float(a))
        sw2 += af * af
        u = exact_quotient_f32(np.float32(abs(a)), m)
        q = _exact_code(u, 1)
        rec = round_fraction(Fraction(q, 15) * mf, 8)
        if a < 0:
            rec = -rec
        se2 += (af - rec) ** 2
    assert got.shape == (1, 2)
    assert math.isclose(got[0, 0], float(sw2), rel_tol=1e-15)
    assert math.isclose(got[0, 1], float(se2), rel_tol=1e-12)


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
def test_error_sums_zero_on_reconstructions(alpha):
    """bfloat16 weights that already are reconstructions come back exactly (the
    row max, a bfloat16 value, reconstructs to itself), so their error sum is 0."""
    rng = np.random.default_rng(31)
    w = (rng.standard_t(4, (6, 64)) * 0.02).astype(np.float32)
    w = torch.from_numpy(w).to(torch.bfloat16).float().numpy()  # bfloat16 values
    w[2] = 0.0
    d = O.bf16_bits_to_f32(O.dequantize(*O.quantize(w, alpha), alpha))
    got = O.error_sums(d, alpha)
    assert np.all(got[:, 1] == 0.0)
    assert np.allclose(got[:, 0], np.sum(d.astype(np.float64) ** 2, axis=1), rtol=1e-14, atol=0)
    assert got[2, 0] == 0.0


def test_error_sums_grow_away_from_reconstructions():
    """Moving a weight off its reconstruction adds exactly that squared gap."""
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 1.0                   # the max: reconstructs exactly
    w[0, 1] = 0.5                   # alpha = 1: code 8, level 8/15
    got = O.error_sums(w, 1.0)
    rec = float(round_fraction(Fraction(8, 15), 8))
    assert math.isclose(got[0, 1], (0.5 - rec) ** 2, rel_tol=1e-15)


# ------------------------------------------------------------------ group-wise scales
#
# The card's stored form keeps one float16 max per group of weights ("技术细节 /
# 存储格式", group sizes 32/64/128/256 in the configuration section).

def _f16_exact(a):
    """Nearest float16 (ties to even) of a nonnegative value, saturated at
    65504, by exact rational rounding (11 significant bits, emin = -14)."""
    fr = min(Fraction(float(a)), Fraction(65504))
    return round_fraction(fr, 11, emin=-14)


def test_group_max_f16_exact_rounding():
    rng = np.random.default_rng(40)
    vals = np.concatenate([
        (rng.random(3000) * np.exp2(rng.integers(-30, 17, 3000))).astype(np.float32),
        np.array([0.0, 65504.0, 65519.0, 65520.0, 1e5, 3e38, 2.0 ** -24, 2.0 ** -25,
                  1.5 * 2.0 ** -25, 2.0 ** -26, 2.0 ** -14, 2.0 ** -15 * 1.5], np.float32),
        # exact midpoints between neighbouring float16 values: ties to even
        (1.0 + (2 * rng.integers(0, 1024, 500) + 1) * 2.0 ** -11).astype(np.float32),
        ((2 * rng.integers(0, 1024, 500) + 1) * 2.0 ** -25).astype(np.float32),
    ])
    gs = 32
    w = np.zeros((len(vals), gs), np.float32)
    w[:, 5] = vals
    w[:, 9] = -vals * np.float32(0.5)
    got = O.group_absmax_f16(w, gs)[:, 0].astype(np.float64)
    ref = np.array([float(_f16_exact(v)) for v in vals])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("gs", [32, 64, 128, 256])
def test_groups_are_row_slabs(gs):
    """With bf16 weights (every group max is a float16 value) the group form
    is the per-row form applied to each slab of gs consecutive columns."""
    w = _to_bf16_values(_rand_rows(41, 6, 512))
    w[2, 64:128] = 0.0                                   # zero groups
    q, s, m16 = O.encode_grouped(w, 0.73, gs)
    pk, sg, _ = O.quantize_grouped(w, 0.73, gs)
    d = O.dequantize_grouped(pk, sg, m16, 0.73, gs)
    for j in range(512 // gs):
        sl = slice(j * gs, (j + 1) * gs)
        qr, sr, mr = O.encode(w[:, sl], 0.73)
        assert np.array_equal(q[:, sl], qr) and np.array_equal(s[:, sl], sr)
        assert np.array_equal(m16[:, j].astype(np.float32), mr)
        pr, sgr, _ = O.quantize(w[:, sl], 0.73)
        assert np.array_equal(d[:, sl], O.dequantize(pr, sgr, mr, 0.73))


@pytest.mark.parametrize("alpha,rule", [
    (1.0, lambda u: min(15, int(np.rint(15 * float(u))))),
    # 15 sqrt(u) >= k - 1/2  <=>  900 u >= (2k-1)^2; codes stop at 15
    (0.5, lambda u: sum(1 for k in range(1, 16) if 900 * u >= (2 * k - 1) ** 2)),
])
def test_group_codes_against_rounded_max(alpha, rule):
    """float32 weights whose group max is no float16 value: u is the binary32
    quotient by the stored (rounded) max, up to just above 1 (code 15)."""
    rng = np.random.default_rng(42)
    gs = 32
    w = (rng.standard_normal((8, 4 * gs)) * 0.02).astype(np.float32)
    w[0, 3] = np.float32(1.0 + 2.0 ** -12)               # rounds down to 1.0
    w[0, 7] = np.float32(-(1.0 + 2.0 ** -13))
    w[1, gs + 1] = np.float32(0.1)                        # rounds up
    q, s, m16 = O.encode_grouped(w, alpha, gs)
    for r in range(w.shape[0]):
        for c in range(w.shape[1]):
            mg = _f16_exact(np.max(np.abs(w[r, (c // gs) * gs:(c // gs + 1) * gs])))
            assert float(m16[r, c // gs]) == float(mg)
            u = Fraction(0) if mg == 0 else Fraction(float(round_fraction(
                Fraction(float(abs(w[r, c]))) / mg, 24)))
            assert q[r, c] == rule(u), (r, c)
            assert s[r, c] == (1 if w[r, c] < 0 else 0)
    assert q[0, 3] == 15 and q[0, 7] == 15 and s[0, 7] == 1


def test_group_zero_tiny_and_saturated_groups():
    gs = 32
    w = np.zeros((3, 3 * gs), np.float32)
    w[0, 1] = 2.0 ** -26                                  # stored max rounds to 0
    w[0, 2] = -(2.0 ** -27)
    w[0, gs] = 2.0 ** -25                                 # a tie: rounds to 0 (even)
    w[0, 2 * gs + 4] = -1.5 * 2.0 ** -25                  # rounds up to 2^-24
    w[1, 5] = 1e5                                         # saturates to 65504
    w[1, 6] = 65504.0
    w[1, 7] = -3e4
    q, s, m16 = O.encode_grouped(w, 0.73, gs)
    assert list(m16[0].astype(np.float64)) == [0.0, 0.0, 2.0 ** -24]
    assert np.all(q[0, :2 * gs] == 0)
    assert s[0, 2] == 1 and s[0, 1] == 0                  # signs still follow w < 0
    # u = 0.75 against the rounded-up max: 15 * 0.75^0.73 = 12.16
    assert q[0, 2 * gs + 4] == 12 and s[0, 2 * gs + 4] == 1
    assert float(m16[1, 0]) == 65504.0 and q[1, 5] == 15 and q[1, 6] == 15
    assert np.all(q[2] == 0) and np.all(s[2] == 0) and np.all(m16[2] == 0)
    pk, sg, _ = O.quantize_grouped(w, 0.73, gs)
    d = O.dequantize_grouped(pk, sg, m16, 0.73, gs)
    assert np.all(d[0, :2 * gs] == 0)                      # +0.0, signs ignored at code 0
    assert np.all(d[2] == 0)
    # q = 15 reconstructs to the stored max itself (bf16 of 65504 is 65536)
    assert d[1, 6] == bf16_bits_of(Fraction(65504))


@pytest.mark.parametrize("alpha,level", [
    (1.0, lambda q: Fraction(q, 15)),
    (0.5, lambda q: Fraction(q, 15) ** 2),
])
def test_group_dequant_exact_rational(alpha, level):
    rng = np.random.default_rng(43)
    gs = 64
    w = (rng.standard_normal((5, 4 * gs)) * np.exp2(rng.integers(-8, 3, (5, 1)))).astype(np.float32)
    pk, sg, m16 = O.quantize_grouped(w, alpha, gs)
    got = O.dequantize_grouped(pk, sg, m16, alpha, gs)
    q, s = O.unpack(pk, sg)
    for r in range(w.shape[0]):
        for c in range(w.shape[1]):
            v = level(int(q[r, c])) * Fraction(float(m16[r, c // gs]))
            if s[r, c] and q[r, c]:
                v = -v
            assert got[r, c] == bf16_bits_of(v), (r, c)


@pytest.mark.parametrize("gs", [32, 128])
def test_group_quantize_dequantize_idempotent(gs):
    w = _to_bf16_values(_rand_rows(44, 6, 256))
    pk, sg, m16 = O.quantize_grouped(w, 0.73, gs)
    d1 = O.dequantize_grouped(pk, sg, m16, 0.73, gs)
    w1 = O.bf16_bits_to_f32(d1)
    pk2, sg2, m2 = O.quantize_grouped(w1, 0.73, gs)
    assert np.array_equal(pk2, pk) and np.array_equal(m2, m16)
    assert np.array_equal(O.dequantize_grouped(pk2, sg2, m2, 0.73, gs), d1)


# ------------------------------------------------------------------ other code widths
#
# The configuration section offers 3, 4, 5 or 6 bits; 2^b - 1 takes the place
# of 15.  The card gives no packing for b != 4; here it is a little-endian bit stream.

def test_bits4_is_the_nibble_form():
    w = _to_bf16_values(_rand_rows(50, 5, 256))
    for alpha in (0.45, 0.73):
        pb, sb, mb = O.quantize_bits(w, alpha, 4)
        p, s, m = O.quantize(w, alpha)
        assert np.array_equal(pb, p) and np.array_equal(sb, s) and np.array_equal(mb, m)
        assert np.array_equal(O.dequantize_bits(pb, sb, mb, alpha, 4), O.dequantize(p, s, m, alpha))


@pytest.mark.parametrize("bits", [3, 4, 5, 6])
def test_bit_stream_packing_by_big_integers(bits):
    """Each row's codes as one Python integer, sum q_i 2^(b i), cut into
    32-bit words from the bottom."""
    rng = np.random.default_rng(51 + bits)
    k = 96
    q = rng.integers(0, 1 << bits, (3, k)).astype(np.uint8)
    got = O.pack_bits(q, bits)
    assert got.shape == (3, k * bits // 32)
    for r in range(3):
        big = sum(int(q[r, i]) << (bits * i) for i in range(k))
        want = [(big >> (32 * j)) & 0xFFFFFFFF for j in range(k * bits // 32)]
        assert got[r].tolist() == want
    assert np.array_equal(O.unpack_bits(got, bits, k), q)


@pytest.mark.parametrize("bits", [3, 5, 6])
def test_bits_alpha_one_is_uniform_rounding(bits):
    """alpha = 1: q = rint((2^b - 1) u), exact in float64."""
    L = (1 << bits) - 1
    w = _rand_rows(52, 6, 64)
    w[0, 3] = np.float32(0.5) * np.abs(w[0]).max()   # u = 1/2: (2^b - 1)/2 is a half -> up
    q, s, m = O.encode_bits(w, 1.0, bits)
    assert np.array_equal(q, _codes_closed_form(w, lambda u: int(np.floor(L * float(u) + 0.5))))
    assert q[0, 3] == (L + 1) // 2
    assert np.array_equal(m, np.max(np.abs(w), axis=1))
    assert np.array_equal(s, (w < 0).astype(np.uint8))


@pytest.mark.parametrize("bits", [3, 5, 6])
def test_bits_half_alpha_exact_rational_codes(bits):
    """alpha = 1/2: L sqrt(u) >= k - 1/2  <=>  4 L^2 u >= (2k - 1)^2."""
    L = (1 << bits) - 1
    w = _rand_rows(53, 5, 64)
    q, _, _ = O.encode_bits(w, 0.5, bits)
    rule = lambda u: sum(1 for kk in range(1, L + 1) if 4 * L * L * u >= (2 * kk - 1) ** 2)
    assert np.array_equal(q, _codes_closed_form(w, rule))


@pytest.mark.parametrize("bits", [3, 5, 6])
@pytest.mark.parametrize("alpha,level", [(1.0, lambda q, L: Fraction(q, L)),
                                         (0.5, lambda q, L: Fraction(q, L) ** 2)])
def test_bits_dequant_exact_rational(bits, alpha, level):
    L = (1 << bits) - 1
    w = _to_bf16_values(_rand_rows(54, 4, 64))
    p, sg, m = O.quantize_bits(w, alpha, bits)
    got = O.dequantize_bits(p, sg, m, alpha, bits)
    q = O.unpack_bits(p, bits, 64)
    _, s = O.unpack(np.zeros((4, 8), np.uint32), sg)
    for r in range(4):
        for c in range(64):
            v = level(int(q[r, c]), L) * Fraction(float(m[r]))
            if s[r, c] and q[r, c]:
                v = -v
            assert got[r, c] == bf16_bits_of(v), (r, c)


@pytest.mark.parametrize("bits", [3, 6])
def test_bits_error_sums_zero_on_reconstructions(bits):
    w = _to_bf16_values(_rand_rows(55, 4, 128))
    p, s, m = O.quantize_bits(w, 0.73, bits)
    w1 = O.bf16_bits_to_f32(O.dequantize_bits(p, s, m, 0.73, bits))
    sums = O.error_sums_bits(w1, 0.73, bits)
    assert np.all(sums[:, 1] == 0.0)
    assert np.allclose(sums[:, 0], np.sum(w1.astype(np.float64) ** 2, axis=1), rtol=0, atol=0)
    # more bits, smaller error (same weights)
    e = [O.error_sums_bits(w, 0.73, b)[:, 1].sum() for b in (3, 4, 5, 6)]
    assert e[0] > e[1] > e[2] > e[3] > 0
