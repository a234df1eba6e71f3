"""GPU parity of the 3/5/6-bit codes (2^b - 1 levels, codes as a bit stream
along k) through the C ABI: codes, signs and scales bit for bit against the
oracle, reconstructions within one bf16 ulp (in practice equal), error sums
within the kernel's stated precision."""
import numpy as np
import pytest
import torch

import oracle as O
from w4a16_linear_amd import workloads as WL
from w4a16_linear_amd.workloads import bf16_bits, u32

from test_gpu_parity import DEV, Guarded, assert_dequant_close, weight_tensor

pytestmark = pytest.mark.gpu

BITS = [3, 5, 6]


def quantize_bits_guarded(opq, w_dev, alpha, bits):
    n, k = w_dev.shape
    gp = Guarded((n, k * bits // 32), torch.int32)
    gsg = Guarded((n, k // 32), torch.int32)
    gm = Guarded((n,), torch.float32)
    bw = opq.BitsWeight(gp.t, gsg.t, gm.t, bits)
    opq.quantize_bits(w_dev, alpha, bits, out=bw)
    torch.cuda.synchronize()
    for g in (gp, gsg, gm):
        g.check()
    return bw


def bits_roundtrip(opq, w_vals, w_dev, alpha, bits):
    bw = quantize_bits_guarded(opq, w_dev, alpha, bits)
    p_ref, s_ref, m_ref = O.quantize_bits(w_vals, alpha, bits)
    assert np.array_equal(bw.scale.cpu().numpy().view(np.uint32), m_ref.view(np.uint32)), "scale"
    for name, got, want in (("packed", u32(bw.packed), p_ref), ("sign", u32(bw.sign), s_ref)):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name} differs at {bad[:5].tolist()} of {bad.shape[0]}"
    n, k = w_dev.shape
    g = Guarded((n, k), torch.bfloat16)
    opq.dequantize(bw, alpha, out=g.t)
    torch.cuda.synchronize()
    g.check()
    d_ref = O.dequantize_bits(p_ref, s_ref, m_ref, alpha, bits)
    q_ref = O.unpack_bits(p_ref, bits, k)
    exact = assert_dequant_close(bf16_bits(g.t), d_ref, q_ref)
    return bw, exact


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
@pytest.mark.parametrize("n,k", [(1, 32), (5, 96), (7, 544), (33, 3840), (3, 16384)])
def test_bits_bf16_shapes(gpu_lib, n, k, alpha, bits):
    w_vals, w_dev = weight_tensor(WL.student_t(1400 + n + k + bits, (n, k)), "bf16")
    bits_roundtrip(gpu_lib, w_vals, w_dev, alpha, bits)


@pytest.mark.parametrize("bits", BITS)
def test_bits_fp32_and_special_rows(gpu_lib, bits):
    from test_gpu_parity import _special_rows
    for dtype in ("f32", "bf16"):
        w_vals, w_dev = weight_tensor(_special_rows(544, dtype), dtype)
        for alpha in (0.3, 0.73, 2.0):
            bits_roundtrip(gpu_lib, w_vals, w_dev, alpha, bits)
    w_vals, w_dev = weight_tensor(WL.normal(1500 + bits, (4, 4096), 0.02), "f32")
    bits_roundtrip(gpu_lib, w_vals, w_dev, 0.73, bits)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
@pytest.mark.parametrize("k", [8192, 2048])
def test_bits_near_decision_points(gpu_lib, bits, alpha, k):
    """Magnitudes within a few binary32 ulps of every row boundary (k = 2048:
    a row to a wave; 8192: a row to a block)."""
    L = (1 << bits) - 1
    t = O.decision_thresholds_f32(alpha, L)
    rows = []
    for m in (np.float32(0.0371), np.float32(1.0)):
        vals = []
        for tk in t:
            ci = int(np.array([tk * m], np.float32).view(np.int32)[0])
            vals.extend(np.arange(ci - 12, ci + 13, dtype=np.int32).view(np.float32).tolist())
        vals = np.array(vals, np.float32)
        vals = vals[(vals >= 0) & (vals <= m)][:k - 1]
        row = np.zeros(k, np.float32)
        row[:len(vals)] = vals
        row[len(vals)] = m
        rows.append(row * np.where(np.arange(k) % 2 == 1, -1.0, 1.0).astype(np.float32))
    w_vals, w_dev = weight_tensor(np.stack(rows), "f32")
    bits_roundtrip(gpu_lib, w_vals, w_dev, alpha, bits)


def test_bits4_equals_the_4bit_calls(gpu_lib):
    opq = gpu_lib
    _, w_dev = weight_tensor(WL.student_t(1600, (40, 544)), "bf16")
    bw = opq.quantize_bits(w_dev, 0.73, 4)
    qw = opq.quantize(w_dev, 0.73)
    assert torch.equal(bw.packed, qw.packed) and torch.equal(bw.sign, qw.sign)
    assert torch.equal(bw.scale, qw.scale)
    assert torch.equal(opq.dequantize(bw, 0.73), opq.dequantize(qw, 0.73))


@pytest.mark.parametrize("bits", BITS)
def test_bits_many_rows_against_sampled_oracle(gpu_lib, bits):
    """More rows than the persistent grid: every block takes several rows."""
    opq = gpu_lib
    n, k = 5003, 3840
    w_vals, w_dev = weight_tensor(WL.student_t(1700 + bits, (n, k)), "bf16")
    bw = opq.quantize_bits(w_dev, 0.73, bits)
    rng = np.random.default_rng(bits)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 200, replace=False)]))
    p_ref, s_ref, m_ref = O.quantize_bits(w_vals[rows], 0.73, bits)
    torch.cuda.synchronize()
    assert np.array_equal(u32(bw.packed)[rows], p_ref)
    assert np.array_equal(u32(bw.sign)[rows], s_ref)
    assert np.array_equal(bw.scale.cpu().numpy()[rows], m_ref)
    sums = opq.error_sums(w_dev, 0.73, bits=bits).cpu().numpy()
    ref = O.error_sums_bits(w_vals[rows], 0.73, bits)
    assert np.allclose(sums[rows], ref, rtol=1e-5, atol=0)


@pytest.mark.parametrize("bits", BITS)
def test_bits_short_rows_past_one_grid(gpu_lib, bits):
    """33000 rows of 96: a row to a wave on a grid of at most 32768 waves, so
    some waves take a second row; every row against the oracle."""
    w = WL.student_t(1760 + bits, (33000, 96))
    w[100] = 0.0
    w_vals, w_dev = weight_tensor(w, "bf16")
    bits_roundtrip(gpu_lib, w_vals, w_dev, 0.73, bits)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("dtype,n,k", [("bf16", 64, 3840), ("f32", 9, 544), ("bf16", 4, 16384)])
def test_bits_error_sums_match_oracle(gpu_lib, bits, dtype, n, k):
    opq = gpu_lib
    w32 = WL.student_t(1800 + n + bits, (n, k))
    w32[0] = 0.0
    w_vals, w_dev = weight_tensor(w32, dtype)
    for alpha in (0.45, 0.73, 1.0):
        got = opq.error_sums(w_dev, alpha, bits=bits).cpu().numpy()
        ref = O.error_sums_bits(w_vals, alpha, bits)
        assert np.all(got[0] == 0.0)
        assert np.allclose(got, ref, rtol=1e-5, atol=0), (alpha, np.max(np.abs(got - ref) / np.maximum(ref, 1e-300)))


def test_bits_snr_grows_with_width(gpu_lib):
    opq = gpu_lib
    _, w_dev = weight_tensor(WL.student_t(1900, (256, 3840)), "bf16")
    snr = [opq.snr_db(w_dev, 0.73, bits=b) for b in (3, 4, 5, 6)]
    assert snr[0] < snr[1] < snr[2] < snr[3]


def test_bits_empty_calls(gpu_lib):
    opq = gpu_lib
    for bits in BITS:
        bw = opq.quantize_bits(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), 0.73, bits)
        assert bw.packed.shape == (0, 2 * bits)
        bw = opq.quantize_bits(torch.empty((3, 0), dtype=torch.bfloat16, device=DEV), 0.73, bits)
        torch.cuda.synchronize()
        assert np.all(bw.scale.cpu().numpy() == 0)
        assert opq.dequantize(bw, 0.73).shape == (3, 0)


# ---------------------------------------------------------------- the linear layer on b-bit codes

def _linear_bits_case(opq, m, n, k, bits, alpha, seed, bias=False, out_dtype=torch.float32,
                      w_dtype="bf16"):
    """opq.linear on b-bit codes against the oracle's reconstruction times x in
    float64: codes bit for bit first, then every output within the tolerance."""
    from test_gpu_parity import Guarded, assert_linear_close
    w_vals, w_dev = weight_tensor(WL.student_t(seed, (n, k)), w_dtype)
    bw = opq.quantize_bits(w_dev, alpha, bits)
    ref = O.quantize_bits(w_vals, alpha, bits)
    assert np.array_equal(u32(bw.packed), ref[0]) and np.array_equal(u32(bw.sign), ref[1])
    d_ref = O.dequantize_bits(*ref, alpha, bits)
    xt = WL.to_bf16(WL.normal(seed + 1, (m, k)))
    b = torch.from_numpy(WL.normal(seed + 2, (n,), 0.1)) if bias else None
    gy = Guarded((m, n), out_dtype)
    opq.linear(xt.to(DEV), bw, alpha, bias=None if b is None else b.to(DEV), out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    y_ref = O.linear(bf16_bits(xt), d_ref, None if b is None else b.numpy())
    y = gy.t.float().cpu().numpy()
    if out_dtype == torch.bfloat16:
        # the float32 result rounded once: within half a bf16 ulp of it, plus the linear bar
        rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
        err = np.abs(y.astype(np.float64) - y_ref)
        assert np.all(err <= 1e-2 * rms + np.abs(y_ref) * 2.0 ** -8 + 1e-30)
        return 0.0
    return assert_linear_close(y, y_ref)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m,n,k", [(1, 48, 96), (8, 256, 256), (16, 300, 544), (32, 1000, 3840),
                                   (33, 17, 160), (64, 520, 1056), (65, 700, 1056),
                                   (300, 513, 3872), (257, 256, 64)])
def test_linear_bits_shapes(gpu_lib, m, n, k, bits):
    """Skinny (m <= 64) and tiled shapes, ragged n and m, k with a final half
    step (k % 64 = 32) and with a final part block (k % 128 != 0)."""
    rel = _linear_bits_case(gpu_lib, m, n, k, bits, 0.73, 2100 + m + n + k + bits)
    print(f"b={bits} m={m} n={n} k={k}: max err / rms = {rel:.2e}")


@pytest.mark.parametrize("bits", BITS)
def test_linear_bits_mid_m_row_slices(gpu_lib, bits):
    """Mid-size m with few weight rows and a long k: the dense product runs on
    slices of up to 64 x rows (ragged last slice), float32 and bf16 output."""
    _linear_bits_case(gpu_lib, 130, 512, 8192, bits, 0.73, 2500 + bits, bias=True)
    _linear_bits_case(gpu_lib, 96, 256, 10240, bits, 0.73, 2510 + bits, bias=True,
                      out_dtype=torch.bfloat16)


@pytest.mark.parametrize("bits", BITS)
def test_linear_bits_bias_bf16_out_fp32_weights(gpu_lib, bits):
    _linear_bits_case(gpu_lib, 40, 300, 512, bits, 0.45, 2200 + bits, bias=True)
    _linear_bits_case(gpu_lib, 130, 300, 512, bits, 1.0, 2210 + bits, bias=True,
                      out_dtype=torch.bfloat16, w_dtype="f32")


@pytest.mark.parametrize("bits", BITS)
def test_linear_bits_full_size(gpu_lib, bits):
    """The skinny workload's weight (3840 x 3840) at every width with x[32, 3840]
    and x[4096, 3840]: every output of both paths within the tolerance."""
    opq = gpu_lib
    from test_gpu_parity import assert_linear_close
    L = WL.config("skinny").layers[0]
    w_vals, w_dev = weight_tensor(L.make_w(), "bf16")
    bw = opq.quantize_bits(w_dev, WL.ALPHA, bits)
    ref = O.quantize_bits(w_vals, WL.ALPHA, bits)
    torch.cuda.synchronize()
    assert np.array_equal(u32(bw.packed), ref[0])
    d_ref = O.dequantize_bits(*ref, WL.ALPHA, bits)
    for m, seed in ((32, 2001), (4096, 3001)):
        xt = WL.to_bf16(WL.normal(seed, (m, L.k)))
        y = opq.linear(xt.to(DEV), bw, WL.ALPHA).cpu().numpy()
        rel = assert_linear_close(y, O.linear(bf16_bits(xt), d_ref))
        print(f"b={bits} m={m}: max err / rms = {rel:.2e}")


def test_linear_bits_workspace_reuse_and_empty(gpu_lib):
    """One workspace serves calls of different widths and shapes in turn; empty
    shapes return the bias (or nothing)."""
    opq = gpu_lib
    ws = torch.empty(opq.linear_workspace_bytes(200, 384, 1024, 6), dtype=torch.uint8, device=DEV)
    outs = []
    for bits, m, n, k in ((6, 200, 384, 1024), (3, 20, 256, 512), (5, 200, 384, 1024)):
        _, w_dev = weight_tensor(WL.student_t(2300 + bits, (n, k)), "bf16")
        bw = opq.quantize_bits(w_dev, 0.73, bits)
        x = WL.to_bf16(WL.normal(2400 + bits, (m, k))).to(DEV)
        y1 = opq.linear(x, bw, 0.73, workspace=ws)
        y2 = opq.linear(x, bw, 0.73)     # the per-device shared workspace
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
        outs.append(y1)
    bw = opq.quantize_bits(torch.zeros((4, 0), dtype=torch.bfloat16, device=DEV), 0.73, 5)
    bias = torch.arange(4, dtype=torch.float32, device=DEV)
    for m in (3, 100):
        y = opq.linear(torch.empty((m, 0), dtype=torch.bfloat16, device=DEV), bw, 0.73, bias=bias)
        assert torch.equal(y.cpu(), bias.cpu().expand(m, 4))
