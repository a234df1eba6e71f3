"""GPU parity: libopq's HIP kernels against the CPU oracle, through the C ABI.

Bars (same inputs, element by element):
  * packed codes, sign words and scales bit-exact;
  * dequantized bfloat16 within 1 ulp (ordered patterns, so -0 and +0 agree),
    and +0.0 for every zero code;
  * linear output max|y - y_ref| <= 1e-2 * rms(y_ref), y_ref the float64 product
    over the oracle's bfloat16 reconstructions.

Every output buffer is a view into a larger pattern-filled allocation; the
margins are checked after each call to catch stray writes.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from w4a16_linear_amd import workloads as WL
from w4a16_linear_amd.workloads import bf16_bits, to_bf16, u32

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MARGIN = 256  # bytes of guard band on each side (keeps 16-byte alignment)
LINEAR_TOL = 1e-2


# ------------------------------------------------------------------ helpers

class Guarded:
    """A tensor view with pattern-filled guard bands before and after it."""

    def __init__(self, shape, dtype):
        self.shape = tuple(shape)
        esz = torch.tensor([], dtype=dtype).element_size()
        self.pad = MARGIN // esz
        numel = int(np.prod(self.shape)) if self.shape else 1
        self.base = torch.empty(numel + 2 * self.pad, dtype=torch.uint8 if esz == 1 else dtype,
                                device=DEV)
        self.base.view(torch.uint8).fill_(0xA5)
        self.t = self.base[self.pad:self.pad + numel].view(self.shape)

    def check(self):
        raw = self.base.view(torch.uint8).cpu().numpy()
        nb = self.pad * self.base.element_size()
        assert np.all(raw[:nb] == 0xA5), "write before the buffer"
        assert np.all(raw[len(raw) - nb:] == 0xA5), "write after the buffer"


def quantize_guarded(opq, w_dev, alpha):
    n, k = w_dev.shape
    gp = Guarded((n, k // 8), torch.int32)
    gs = Guarded((n, k // 32), torch.int32)
    gm = Guarded((n,), torch.float32)
    qw = opq.QuantizedWeight(gp.t, gs.t, gm.t)
    opq.quantize(w_dev, alpha, out=qw)
    torch.cuda.synchronize()
    for g in (gp, gs, gm):
        g.check()
    return qw


def dequantize_guarded(opq, qw, alpha):
    n, k = qw.shape
    g = Guarded((n, k), torch.bfloat16)
    opq.dequantize(qw, alpha, out=g.t)
    torch.cuda.synchronize()
    g.check()
    return g.t


def ordered(bits):
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def assert_quant_equal(qw, ref, rows=None):
    p_ref, s_ref, m_ref = ref
    sel = slice(None) if rows is None else rows
    p = u32(qw.packed)[sel]
    s = u32(qw.sign)[sel]
    m = qw.scale.cpu().numpy()[sel]
    assert np.array_equal(m.view(np.uint32), m_ref.view(np.uint32)), "scale"
    bad = np.argwhere(p != p_ref)
    assert bad.size == 0, f"packed differs at {bad[:5].tolist()} of {bad.shape[0]}"
    bad = np.argwhere(s != s_ref)
    assert bad.size == 0, f"sign differs at {bad[:5].tolist()} of {bad.shape[0]}"


def assert_dequant_close(d_bits, ref_bits, q_ref):
    dist = np.abs(ordered(d_bits) - ordered(ref_bits))
    assert dist.max(initial=0) <= 1, f"max ulp distance {dist.max()}"
    zero = q_ref == 0
    assert np.all(d_bits[zero] == 0), "code 0 must give +0.0"
    return float(np.mean(dist == 0)) if dist.size else 1.0


def assert_linear_close(y, y_ref):
    rms = math.sqrt(float(np.mean(y_ref * y_ref))) if y_ref.size else 0.0
    err = float(np.max(np.abs(y.astype(np.float64) - y_ref))) if y_ref.size else 0.0
    assert err <= LINEAR_TOL * rms + 1e-30, f"max err {err:.3e} > {LINEAR_TOL} * rms {rms:.3e}"
    return err / rms if rms else 0.0


def weight_tensor(w32, dtype):
    """Host float32 values -> (exact float32 values of the stored dtype, device tensor)."""
    if dtype == "bf16":
        t = to_bf16(w32)
        return O.bf16_bits_to_f32(bf16_bits(t)), t.to(DEV)
    return np.ascontiguousarray(w32, np.float32), torch.from_numpy(np.ascontiguousarray(w32)).to(DEV)


def full_roundtrip(opq, w_vals, w_dev, alpha):
    """Quantize + dequantize on the GPU and in the oracle; compare everything."""
    qw = quantize_guarded(opq, w_dev, alpha)
    ref = O.quantize(w_vals, alpha)
    assert_quant_equal(qw, ref)
    d = dequantize_guarded(opq, qw, alpha)
    d_ref = O.dequantize(*ref, alpha)
    q_ref, _ = O.unpack(ref[0], ref[1])
    assert_dequant_close(bf16_bits(d), d_ref, q_ref)
    return qw, ref, d_ref


# ------------------------------------------------------------------ tiny config (whole path)

def test_tiny_config_whole_path(gpu_lib):
    opq = gpu_lib
    cfg = WL.config("tiny")
    L = cfg.layers[0]
    w_vals, w_dev = weight_tensor(L.make_w(), L.w_dtype)
    qw, ref, d_ref = full_roundtrip(opq, w_vals, w_dev, WL.ALPHA)
    xt = to_bf16(L.make_x())
    gy = Guarded((L.m, L.n), torch.float32)
    opq.linear(xt.to(DEV), qw, WL.ALPHA, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    y_ref = O.linear(bf16_bits(xt), d_ref)
    assert_linear_close(gy.t.cpu().numpy(), y_ref)


# ------------------------------------------------------------------ quantize / dequantize edge cases

SHAPES = [(1, 32), (5, 96), (7, 544), (3, 2048), (3, 2080), (33, 3840), (3, 10240), (2, 16384),
          (2, 16416), (3, 20480)]


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
@pytest.mark.parametrize("n,k", SHAPES)
def test_quantize_bf16_shapes(gpu_lib, n, k, alpha):
    w = WL.student_t(100 + n + k, (n, k))
    w_vals, w_dev = weight_tensor(w, "bf16")
    full_roundtrip(gpu_lib, w_vals, w_dev, alpha)


@pytest.mark.parametrize("n,k", [(3, 256), (5, 2048), (4, 2080), (4, 4096), (2, 8192), (2, 8224),
                                 (3, 12288), (2, 16416), (2, 20480)])
def test_quantize_fp32_shapes(gpu_lib, n, k):
    w = WL.normal(200 + k, (n, k), 0.02)
    w_vals, w_dev = weight_tensor(w, "f32")
    full_roundtrip(gpu_lib, w_vals, w_dev, 0.73)


@pytest.mark.parametrize("dtype,n,k", [("bf16", 9001, 96), ("f32", 8500, 544), ("bf16", 33000, 96),
                                       ("f32", 33000, 544), ("bf16", 33000, 2048)])
def test_quantize_short_rows_past_one_grid(gpu_lib, dtype, n, k):
    """Rows of up to 2048 elements go one to a wave, on a grid of at most 32768
    waves: more rows than that make waves take a second row (its loads issued
    after the first row's stores).  9001 and 8500 rows: one row per wave."""
    w = WL.student_t(400 + n, (n, k))
    w[n // 2] = 0.0
    w_vals, w_dev = weight_tensor(w, dtype)
    full_roundtrip(gpu_lib, w_vals, w_dev, 0.73)


def _special_rows(k, dtype):
    rng = np.random.default_rng(7)
    rows = []
    rows.append(np.zeros(k, np.float32))                                    # all zero
    r = np.zeros(k, np.float32); r[::3] = -0.0; rows.append(r)              # signed zeros
    r = (rng.standard_normal(k) * 0.02).astype(np.float32); r[k // 2] = -1.5; rows.append(r)
    rows.append((rng.standard_normal(k) * 1e-39).astype(np.float32))        # subnormal scale
    rows.append((rng.standard_normal(k) * 1e37).astype(np.float32))         # huge scale
    rows.append(np.full(k, -0.25, np.float32))                              # constant magnitude
    r = np.zeros(k, np.float32); r[5] = 3.0; r[6] = -1e-30; rows.append(r)  # tiny negative
    rows.append(np.linspace(-1, 1, k).astype(np.float32))
    r = (rng.standard_normal(k) * 0.02).astype(np.float32); r[r < 0] = -0.0; rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("alpha", [0.1, 0.45, 0.73, 1.0, 2.0, 5.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_special_rows(gpu_lib, dtype, alpha):
    w = _special_rows(544, dtype)
    w_vals, w_dev = weight_tensor(w, dtype)
    full_roundtrip(gpu_lib, w_vals, w_dev, alpha)


@pytest.mark.parametrize("alpha", [0.03, 100.0])
@pytest.mark.parametrize("dtype,n,k", [("bf16", 5, 96), ("bf16", 7, 544), ("f32", 9, 3840),
                                       ("bf16", 3, 8224), ("f32", 2, 16416), ("bf16", 2, 16416)])
def test_quantize_alpha_without_bucket_grid(gpu_lib, alpha, dtype, n, k):
    """Alphas whose decision points no bucket grid separates (at 0.03 the first
    lies below the normal binary32 range, at 100 all crowd below 1): the
    per-row threshold kernels, with the levels' subnormal reconstructions at
    0.03, against the oracle; k > 16384 streams the row twice."""
    w = WL.student_t(300 + n + k, (n, k))
    w_vals, w_dev = weight_tensor(w, dtype)
    full_roundtrip(gpu_lib, w_vals, w_dev, alpha)


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
def test_quantize_near_decision_points(gpu_lib, alpha):
    """Magnitudes within a few binary32 ulps of every row boundary A_k."""
    k = 1024
    t = O.decision_thresholds_f32(alpha)
    rows = []
    for m in (np.float32(0.0371), np.float32(1.0), np.float32(3.1e-3)):
        vals = []
        for tk in t:
            ci = int(np.array([tk * m], np.float32).view(np.int32)[0])
            steps = np.arange(ci - 24, ci + 25, dtype=np.int32)
            vals.extend(steps.view(np.float32).tolist())
        vals = np.array(vals, np.float32)
        vals = vals[(vals >= 0) & (vals <= m)]
        row = np.zeros(k, np.float32)
        row[:len(vals)] = vals
        row[len(vals)] = m
        sgn = np.where(np.arange(k) % 2 == 1, -1.0, 1.0).astype(np.float32)
        rows.append(row * sgn)
    w = np.stack(rows)
    w_vals, w_dev = weight_tensor(w, "f32")
    full_roundtrip(gpu_lib, w_vals, w_dev, alpha)


def test_empty_calls(gpu_lib):
    opq = gpu_lib
    w = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    qw = opq.quantize(w, 0.73)
    assert qw.packed.shape == (0, 8)
    w = torch.empty((3, 0), dtype=torch.bfloat16, device=DEV)
    qw = opq.quantize(w, 0.73)
    torch.cuda.synchronize()
    assert np.all(qw.scale.cpu().numpy() == 0)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    qw = opq.quantize(to_bf16(WL.normal(1, (16, 64), 0.02)).to(DEV), 0.73)
    y = opq.linear(x, qw, 0.73)
    assert y.shape == (0, 16)
    # k = 0: y = bias
    qw0 = opq.quantize(torch.empty((16, 0), dtype=torch.bfloat16, device=DEV), 0.73)
    bias = torch.arange(16, dtype=torch.float32, device=DEV)
    for m in (4, 200):
        y = opq.linear(torch.empty((m, 0), dtype=torch.bfloat16, device=DEV), qw0, 0.73, bias=bias)
        assert torch.equal(y.cpu(), bias.cpu().expand(m, 16))


# ------------------------------------------------------------------ linear edge cases

@pytest.mark.parametrize("m", [1, 8, 16, 33, 64, 65, 128, 130, 257])
@pytest.mark.parametrize("n,k", [(16, 32), (100, 256), (300, 544), (129, 96)])
def test_linear_shapes(gpu_lib, m, n, k):
    opq = gpu_lib
    w_vals, w_dev = weight_tensor(WL.student_t(300 + n, (n, k)), "bf16")
    qw = quantize_guarded(opq, w_dev, 0.73)
    ref = O.quantize(w_vals, 0.73)
    assert_quant_equal(qw, ref)
    d_ref = O.dequantize(*ref, 0.73)
    xt = to_bf16(WL.normal(400 + m, (m, k)))
    bias = WL.normal(500 + n, (n,), 0.5)
    gy = Guarded((m, n), torch.float32)
    opq.linear(xt.to(DEV), qw, 0.73, bias=torch.from_numpy(bias).to(DEV), out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    y_ref = O.linear(bf16_bits(xt), d_ref, bias)
    assert_linear_close(gy.t.cpu().numpy(), y_ref)


@pytest.mark.parametrize("m,n,k,out_dtype", [(130, 1024, 8192, torch.float32),
                                             (96, 512, 10240, torch.bfloat16),
                                             (257, 768, 6144, torch.float32),
                                             (65, 256, 16384, torch.bfloat16)])
def test_linear_mid_m_row_slices(gpu_lib, m, n, k, out_dtype):
    """Mid-size m with few weight rows and a long k: a handful of 256-row
    tiles would each walk all of k, so the rows go through the skinny kernel
    in slices of up to 64 (the last one ragged).  Every output against the
    oracle, nothing written outside y, bf16 output the float32 one rounded."""
    opq = gpu_lib
    w_vals, w_dev = weight_tensor(WL.student_t(800 + n + k, (n, k)), "bf16")
    qw = quantize_guarded(opq, w_dev, 0.73)
    ref = O.quantize(w_vals, 0.73)
    assert_quant_equal(qw, ref)
    d_ref = O.dequantize(*ref, 0.73)
    xt = to_bf16(WL.normal(900 + m, (m, k)))
    bias = torch.from_numpy(WL.normal(950 + n, (n,), 0.5)).to(DEV)
    gy = Guarded((m, n), torch.float32)
    opq.linear(xt.to(DEV), qw, 0.73, bias=bias, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    assert_linear_close(gy.t.cpu().numpy(), O.linear(bf16_bits(xt), d_ref, bias.cpu().numpy()))
    if out_dtype == torch.bfloat16:
        gb = Guarded((m, n), torch.bfloat16)
        opq.linear(xt.to(DEV), qw, 0.73, bias=bias, out=gb.t)
        torch.cuda.synchronize()
        gb.check()
        b32 = gy.t.cpu().numpy().view(np.uint32).astype(np.uint64)
        assert np.array_equal(bf16_bits(gb.t.cpu()),
                              ((b32 + 0x7FFF + ((b32 >> 16) & 1)) >> 16).astype(np.uint16))


@pytest.mark.parametrize("alpha", [0.03, 100.0])
@pytest.mark.parametrize("m", [8, 300])
def test_linear_alpha_without_bucket_grid(gpu_lib, m, alpha):
    """The linear layer's on-chip tables at alphas far from the usual range
    (subnormal reconstructions at 0.03, levels crowded near 1 at 100): skinny
    and tiled paths against the oracle's reconstruction."""
    opq = gpu_lib
    n, k = 200, 544
    w_vals, w_dev = weight_tensor(WL.student_t(600 + n, (n, k)), "bf16")
    qw = quantize_guarded(opq, w_dev, alpha)
    ref = O.quantize(w_vals, alpha)
    assert_quant_equal(qw, ref)
    d_ref = O.dequantize(*ref, alpha)
    xt = to_bf16(WL.normal(700 + m, (m, k)))
    gy = Guarded((m, n), torch.float32)
    opq.linear(xt.to(DEV), qw, alpha, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    assert_linear_close(gy.t.cpu().numpy(), O.linear(bf16_bits(xt), d_ref))


def test_linear_one_hot_rows_pick_weights(gpu_lib):
    """x = identity rows: y[:, n] is the reconstruction W'[n, :] itself."""
    opq = gpu_lib
    k, n = 256, 96
    w_vals, w_dev = weight_tensor(WL.student_t(600, (n, k)), "bf16")
    qw = opq.quantize(w_dev, 0.73)
    d = opq.dequantize(qw, 0.73)
    for m in (k, 64):
        x = torch.zeros((m, k), dtype=torch.bfloat16)
        x[torch.arange(m), torch.arange(m)] = 1.0
        y = opq.linear(x.to(DEV), qw, 0.73).cpu()
        assert torch.equal(y, d.cpu().float()[:, :m].T.contiguous())


@pytest.mark.parametrize("m,n,k", [(1, 200, 4096), (17, 64, 8192), (32, 130, 2080),
                                   (48, 1000, 1024), (64, 64, 65536), (64, 4000, 96)])
def test_linear_skinny_long_k(gpu_lib, m, n, k):
    """Skinny shapes with many k blocks per wave, ragged n and m, k up to the limit."""
    opq = gpu_lib
    w_vals, w_dev = weight_tensor(WL.student_t(700 + n, (n, k)), "bf16")
    qw = opq.quantize(w_dev, 0.73)
    ref = O.quantize(w_vals, 0.73)
    torch.cuda.synchronize()
    assert_quant_equal(qw, ref)
    xt = to_bf16(WL.normal(800 + m, (m, k)))
    gy = Guarded((m, n), torch.float32)
    opq.linear(xt.to(DEV), qw, 0.73, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    y_ref = O.linear(bf16_bits(xt), O.dequantize(*ref, 0.73))
    assert_linear_close(gy.t.cpu().numpy(), y_ref)


@pytest.mark.parametrize("m,n,k", [(300, 3840, 3840), (1024, 3840, 3840), (2048, 1000, 4096),
                                   (700, 256, 10240), (200, 3840, 3840), (130, 1024, 8192)])
def test_linear_split_k_tiles(gpu_lib, m, n, k):
    """The tiled layer with k split over slices (few 256 x 256 tiles, long k):
    every output against the oracle (with bias), bf16 output the float32 one
    rounded, nothing written past the workspace the call asks for, and the
    same bits twice."""
    opq = gpu_lib
    need = opq.linear_workspace_bytes(m, n, k)
    assert need > 0 and need % 256 == 0
    w_vals, w_dev = weight_tensor(WL.student_t(1900 + n + k, (n, k)), "bf16")
    qw = opq.quantize(w_dev, 0.73)
    ref = O.quantize(w_vals, 0.73)
    torch.cuda.synchronize()
    assert_quant_equal(qw, ref)
    xt = to_bf16(WL.normal(2000 + m, (m, k)))
    bias = WL.normal(2100 + n, (n,), 0.5)
    bias_dev = torch.from_numpy(bias).to(DEV)
    ws = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device=DEV)
    gy = Guarded((m, n), torch.float32)
    opq.linear(xt.to(DEV), qw, 0.73, bias=bias_dev, out=gy.t, workspace=ws)
    torch.cuda.synchronize()
    gy.check()
    assert bool((ws[need:] == 0xA5).all()), "written past the workspace size"
    y1 = gy.t.cpu().numpy()
    assert_linear_close(y1, O.linear(bf16_bits(xt), O.dequantize(*ref, 0.73), bias))
    gy2 = Guarded((m, n), torch.float32)
    opq.linear(xt.to(DEV), qw, 0.73, bias=bias_dev, out=gy2.t, workspace=ws)
    gb = Guarded((m, n), torch.bfloat16)
    opq.linear(xt.to(DEV), qw, 0.73, bias=bias_dev, out=gb.t, workspace=ws)
    torch.cuda.synchronize()
    gy2.check()
    gb.check()
    assert np.array_equal(gy2.t.cpu().numpy().view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(bf16_bits(gb.t.cpu()), _bf16_rne_bits(y1))


def _bf16_rne_bits(y32):
    b = y32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("m,n,k", [(8, 300, 544), (32, 3840, 3840), (200, 300, 544)])
def test_linear_repeatable_and_bf16_out(gpu_lib, m, n, k):
    """Same call twice gives the same bits (fixed sum order; a workspace passed
    in stays reusable), and bfloat16 output is the float32 output rounded to
    nearest even."""
    opq = gpu_lib
    _, w_dev = weight_tensor(WL.student_t(900 + n, (n, k)), "bf16")
    qw = opq.quantize(w_dev, 0.73)
    x = to_bf16(WL.normal(901 + m, (m, k))).to(DEV)
    bias = torch.from_numpy(WL.normal(902, (n,), 0.5)).to(DEV)
    need = max(opq.linear_workspace_bytes(m, n, k), opq.linear_workspace_bytes(5, n, k), 16)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    y1 = opq.linear(x, qw, 0.73, bias=bias, workspace=ws).cpu().numpy()
    # another shape through the same workspace in between
    x_small = to_bf16(WL.normal(903, (5, k))).to(DEV)
    opq.linear(x_small, qw, 0.73, workspace=ws)
    y2 = opq.linear(x, qw, 0.73, bias=bias, workspace=ws).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    gb = Guarded((m, n), torch.bfloat16)
    opq.linear(x, qw, 0.73, bias=bias, out=gb.t, workspace=ws)
    torch.cuda.synchronize()
    gb.check()
    assert np.array_equal(bf16_bits(gb.t.cpu()), _bf16_rne_bits(y1))


# ------------------------------------------------------------------ past one launch's grid

def test_dequantize_rows_past_one_grid(gpu_lib):
    """2^25 + 1000 rows of k = 32: the per-row and 3-bit dequantizers (a wave
    per row segment) need two launches to stay within the 32-bit grid; rows on
    both sides of the split against the oracle.  Weights drawn on the GPU."""
    opq = gpu_lib
    n, k = (1 << 25) + 1000, 32
    g = torch.Generator(device=DEV)
    g.manual_seed(2024)
    w = (torch.randn((n, k), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    rows = np.array([0, 1, (1 << 25) - 2, (1 << 25) - 1, 1 << 25, (1 << 25) + 1, n - 1])
    w_rows = bf16_bits(w[torch.from_numpy(rows).to(DEV)].cpu())
    w_vals = (w_rows.astype(np.uint32) << 16).view(np.float32)
    qw = opq.quantize(w, 0.73)
    d = opq.dequantize(qw, 0.73)
    idx = torch.from_numpy(rows).to(DEV)
    ref = O.quantize(w_vals, 0.73)
    torch.cuda.synchronize()
    assert np.array_equal(u32(qw.packed[idx].cpu()), ref[0])
    assert_dequant_close(bf16_bits(d[idx].cpu()), O.dequantize(*ref, 0.73), O.unpack(ref[0], ref[1])[0])
    del qw, d
    bw = opq.quantize_bits(w, 0.73, 3)
    d = opq.dequantize(bw, 0.73)
    ref = O.quantize_bits(w_vals, 0.73, 3)
    torch.cuda.synchronize()
    assert np.array_equal(u32(bw.packed[idx].cpu()), ref[0])
    assert_dequant_close(bf16_bits(d[idx].cpu()), O.dequantize_bits(*ref, 0.73, 3),
                         O.unpack_bits(ref[0], 3, k))


# ------------------------------------------------------------------ full-size configs

def _sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(count, n), replace=False)]))


def _check_layer(opq, L, alpha, with_linear):
    """One layer at its full size: packed codes, sign words and scales of every
    row bit for bit, every reconstructed weight within 1 ulp, and (with the
    paired activation) every element of y within the linear tolerance."""
    w32 = L.make_w()
    w_vals, w_dev = weight_tensor(w32, L.w_dtype)
    del w32
    qw = opq.quantize(w_dev, alpha)
    ref = O.quantize(w_vals, alpha)
    torch.cuda.synchronize()
    assert_quant_equal(qw, ref)
    del w_vals
    d = opq.dequantize(qw, alpha)
    d_ref = O.dequantize(*ref, alpha)
    q_ref, _ = O.unpack(ref[0], ref[1])
    assert_dequant_close(bf16_bits(d), d_ref, q_ref)
    del d, q_ref, ref
    if not with_linear:
        return None
    xt = to_bf16(L.make_x())
    y = opq.linear(xt.to(DEV), qw, alpha).cpu().numpy()
    y_ref = O.linear(bf16_bits(xt), d_ref)
    return assert_linear_close(y, y_ref)


@pytest.mark.parametrize("dtype,n,k", [("bf16", 6007, 3840), ("bf16", 8200, 5120),
                                       ("bf16", 8200, 3840), ("f32", 6100, 2080)])
def test_quantize_rows_around_block_per_row_bound(gpu_lib, dtype, n, k):
    """Row counts below and above the bound up to which each row gets a block
    of its own (four times the blocks resident at once; past it blocks stride
    over rows; bfloat16 rows of up to 4096 elements go one to a wave from 8192
    rows on): codes, signs and scales at sampled rows equal the oracle's."""
    opq = gpu_lib
    w32 = WL.student_t(500 + n, (n, k))
    w_vals, w_dev = weight_tensor(w32, dtype)
    del w32
    qw = opq.quantize(w_dev, WL.ALPHA)
    rows = _sample_rows(n, 256, n + k)
    ref_rows = O.quantize(w_vals[rows], WL.ALPHA)
    torch.cuda.synchronize()
    assert_quant_equal(qw, ref_rows, rows)


@pytest.mark.parametrize("n,k", [(8191, 3008), (8192, 3008), (9000, 4096), (8192, 2080)])
def test_quantize_bf16_rows_one_to_a_wave_bound(gpu_lib, n, k):
    """bfloat16 rows of 2049..4096 elements go one to a wave from 8192 rows on
    and get a block each below that: both sides of the bound, whole and ragged
    last chunks, a zero row and a row of signed zeros among the sampled rows;
    codes, signs and scales there equal the oracle's."""
    opq = gpu_lib
    w32 = WL.student_t(600 + n + k, (n, k))
    w32[n // 2] = 0.0
    w32[n // 3, ::2] = -0.0
    w_vals, w_dev = weight_tensor(w32, "bf16")
    del w32
    qw = opq.quantize(w_dev, WL.ALPHA)
    rows = np.union1d(_sample_rows(n, 256, n + k), [n // 3, n // 2])
    ref_rows = O.quantize(w_vals[rows], WL.ALPHA)
    torch.cuda.synchronize()
    assert_quant_equal(qw, ref_rows, rows)


@pytest.mark.parametrize("key", ["skinny", "qkv", "ffn"])
def test_config_full_size(gpu_lib, key):
    """Every row and every output of the skinny, QKV and FFN workloads."""
    cfg = WL.config(key)
    for L in cfg.layers:
        rel = _check_layer(gpu_lib, L, WL.ALPHA, with_linear=True)
        print(f"{key}/{L.name}: linear max err / rms = {rel:.2e}", flush=True)


@pytest.mark.parametrize("alpha", WL.ALPHAS_SWEEP)
def test_model_layer_shapes(gpu_lib, alpha):
    """The four block shapes of the whole-model workload drawn by the host
    recipe (first and last block), every row."""
    cfg = WL.config("model")
    for L in cfg.layers[:4] + cfg.layers[-4:]:
        _check_layer(gpu_lib, L, alpha, with_linear=False)


@pytest.mark.parametrize("first_block", range(0, WL.BLOCKS, 5))
def test_model_all_layers_device_weights(gpu_lib, first_block):
    """All 120 layers of the whole-model pass (five blocks per case) at each of
    its three alphas, on the very weights the benchmark quantizes (drawn on the
    device per layer seed): codes, signs and scales of sampled rows bit for bit
    against the oracle, their reconstructions within 1 ulp.  Rows: the first,
    the last and 24 more per layer, a different draw for every layer and alpha."""
    opq = gpu_lib
    rng = np.random.default_rng(5555 + first_block)
    for b in range(first_block, min(first_block + 5, WL.BLOCKS)):
        for i, (name, n, k) in enumerate(WL.BLOCK_LAYERS):
            seed = WL.model_seed(b, i)
            w_dev = WL.student_t_device(seed, (n, k), DEV)
            for alpha in WL.ALPHAS_SWEEP:
                qw = opq.quantize(w_dev, alpha)
                d = opq.dequantize(qw, alpha)
                rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 24, replace=False)]))
                ridx = torch.from_numpy(rows).to(DEV)
                w_rows = O.bf16_bits_to_f32(bf16_bits(w_dev[ridx]))
                ref = O.quantize(w_rows, alpha)
                got = opq.QuantizedWeight(qw.packed[ridx], qw.sign[ridx], qw.scale[ridx])
                assert_quant_equal(got, ref)
                q_ref, _ = O.unpack(ref[0], ref[1])
                assert_dequant_close(bf16_bits(d[ridx]), O.dequantize(*ref, alpha), q_ref)
                del qw, d
            del w_dev
        print(f"block {b}: 4 layers x {len(WL.ALPHAS_SWEEP)} alphas ok", flush=True)


# ------------------------------------------------------------------ error sums (alpha sweep)

# Row sums: binary32 per lane, then across the wave (rows of up to 2048
# elements: one wave per row, at most 32 terms per lane) or across the block's
# four waves in double (longer rows, at most 64 terms per lane per chunk);
# nonnegative terms, so the relative error stays far below 1e-5.
ERR_RTOL = 1e-5


def _assert_sums_close(got, ref):
    got = np.asarray(got, np.float64)
    scale_ = np.maximum(np.abs(ref), 1e-300)
    bad = np.abs(got - ref) > ERR_RTOL * scale_ + 1e-30
    assert not bad.any(), f"rows {np.argwhere(bad)[:5].ravel().tolist()}: {got[bad][:4]} vs {ref[bad][:4]}"


@pytest.mark.parametrize("alpha", [0.3, 0.45, 0.73, 1.0])
@pytest.mark.parametrize("dtype,n,k", [("bf16", 64, 3840), ("bf16", 33, 96), ("f32", 40, 544),
                                       ("bf16", 8, 16384), ("f32", 5, 32)])
def test_error_sums_match_oracle(gpu_lib, alpha, dtype, n, k):
    opq = gpu_lib
    w32 = WL.student_t(1000 + n + k, (n, k))
    w32[0] = 0.0                       # an all-zero row
    if n > 3:
        w32[3] = 0.0
        w32[3, k // 2] = -0.5          # a row with a single (negative) weight
    w_vals, w_dev = weight_tensor(w32, dtype)
    got = opq.error_sums(w_dev, alpha).cpu().numpy()
    ref = O.error_sums(w_vals, alpha)
    _assert_sums_close(got, ref)
    assert np.all(got[0] == 0.0)


@pytest.mark.parametrize("dtype,n,k", [("bf16", 6007, 3840), ("bf16", 4099, 10240), ("f32", 2500, 1056),
                                       ("bf16", 9001, 1024), ("bf16", 9001, 2048)])
def test_error_sums_agree_with_stored_form(gpu_lib, dtype, n, k):
    """More rows than the persistent grid (each block takes several rows, odd
    and even counts): the fused sums equal those of the library's own quantize +
    dequantize at every row, and the oracle's at sampled rows."""
    opq = gpu_lib
    w32 = WL.student_t(77 + n, (n, k))
    w32[n // 3] = 0.0
    w_vals, w_dev = weight_tensor(w32, dtype)
    rows = _sample_rows(n, 24, n)
    for alpha in (0.45, 0.73, 1.0):
        got = opq.error_sums(w_dev, alpha).cpu().numpy()
        d = opq.dequantize(opq.quantize(w_dev, alpha), alpha).double()
        wd = w_dev.double()
        ref = torch.stack([(wd * wd).sum(1), ((wd - d) ** 2).sum(1)], 1).cpu().numpy()
        _assert_sums_close(got, ref)
        _assert_sums_close(got[rows], O.error_sums(w_vals[rows], alpha))
        del d, wd


def test_error_sums_empty(gpu_lib):
    opq = gpu_lib
    z = torch.empty((7, 0), dtype=torch.bfloat16, device=DEV)
    out = torch.full((7, 2), -1.0, dtype=torch.float64, device=DEV)
    assert np.all(opq.error_sums(z, 0.73, out=out).cpu().numpy() == 0.0)
    assert opq.error_sums(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), 0.73).shape == (0, 2)


def test_concurrent_streams_different_alphas(gpu_lib):
    """Calls with different alphas enqueued on two streams at once give the
    results each gives alone (no state shared between calls)."""
    opq = gpu_lib
    _, w_dev = weight_tensor(WL.student_t(950, (512, 3840)), "bf16")
    x = to_bf16(WL.normal(951, (200, 3840))).to(DEV)
    ref = {}
    for a in (0.45, 1.0):
        qw = opq.quantize(w_dev, a)
        ref[a] = (u32(qw.packed), opq.dequantize(qw, a).cpu(), opq.linear(x, qw, a).cpu(),
                  opq.error_sums(w_dev, a).cpu())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    outs = {}
    torch.cuda.synchronize()
    for rep in range(3):
        for a, s in zip((0.45, 1.0), streams):
            with torch.cuda.stream(s):
                qw = opq.quantize(w_dev, a)
                ws = torch.zeros(max(opq.linear_workspace_bytes(200, 512, 3840), 16),
                                 dtype=torch.uint8, device=DEV)
                outs[a] = (qw, opq.dequantize(qw, a), opq.linear(x, qw, a, workspace=ws),
                           opq.error_sums(w_dev, a))
        torch.cuda.synchronize()
        for a in (0.45, 1.0):
            qw, d, y, e = outs[a]
            assert np.array_equal(u32(qw.packed), ref[a][0])
            assert torch.equal(d.cpu(), ref[a][1])
            assert torch.equal(y.cpu(), ref[a][2])
            assert torch.equal(e.cpu(), ref[a][3])
