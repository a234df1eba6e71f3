"""GPU parity of the group-wise stored form (one float16 max per group of
weights along k, the card's own format) through the C ABI: codes, signs and
stored maxima bit for bit against the oracle, the bf16 reconstruction bit for
bit, and the linear layer within max|y - y_ref| <= 1e-2 rms(y_ref)."""
import numpy as np
import pytest
import torch

import oracle as O
from w4a16_linear_amd import workloads as WL
from w4a16_linear_amd.workloads import bf16_bits, to_bf16, u32

from test_gpu_parity import DEV, Guarded, assert_linear_close, weight_tensor

pytestmark = pytest.mark.gpu

GROUPS = [32, 64, 128, 256]


def quantize_grouped_guarded(opq, w_dev, alpha, gs):
    n, k = w_dev.shape
    gp = Guarded((n, k // 8), torch.int32)
    gsg = Guarded((n, k // 32), torch.int32)
    gm = Guarded((n, k // gs), torch.float16)
    gw = opq.GroupedWeight(gp.t, gsg.t, gm.t, gs)
    opq.quantize_grouped(w_dev, alpha, gs, out=gw)
    torch.cuda.synchronize()
    for g in (gp, gsg, gm):
        g.check()
    return gw


def assert_grouped_equal(gw, ref, rows=None):
    p_ref, s_ref, m_ref = ref
    sel = slice(None) if rows is None else rows
    m = gw.scale16.cpu().numpy()[sel]
    bad = np.argwhere(m.view(np.uint16) != np.asarray(m_ref, np.float16).view(np.uint16))
    assert bad.size == 0, f"scale16 differs at {bad[:5].tolist()}"
    for name, got, want in (("packed", u32(gw.packed)[sel], p_ref), ("sign", u32(gw.sign)[sel], s_ref)):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name} differs at {bad[:5].tolist()} of {bad.shape[0]}"


def grouped_roundtrip(opq, w_vals, w_dev, alpha, gs):
    gw = quantize_grouped_guarded(opq, w_dev, alpha, gs)
    ref = O.quantize_grouped(w_vals, alpha, gs)
    assert_grouped_equal(gw, ref)
    n, k = w_dev.shape
    g = Guarded((n, k), torch.bfloat16)
    opq.dequantize(gw, alpha, out=g.t)
    torch.cuda.synchronize()
    g.check()
    d_ref = O.dequantize_grouped(*ref, alpha, gs)
    bad = np.argwhere(bf16_bits(g.t) != d_ref)
    assert bad.size == 0, f"dequant differs at {bad[:5].tolist()} of {bad.shape[0]}"
    return gw, ref, d_ref


@pytest.mark.parametrize("gs", GROUPS)
@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
@pytest.mark.parametrize("n,k", [(1, 256), (37, 512), (5, 768), (33, 3840), (2, 20480)])
def test_grouped_bf16_shapes(gpu_lib, n, k, alpha, gs):
    if k % gs:
        pytest.skip("group does not divide k")
    w_vals, w_dev = weight_tensor(WL.student_t(700 + n + k, (n, k)), "bf16")
    grouped_roundtrip(gpu_lib, w_vals, w_dev, alpha, gs)


@pytest.mark.parametrize("gs", GROUPS)
@pytest.mark.parametrize("n,k", [(3, 256), (7, 96 * 32), (1, 32 * 256 + 256)])
def test_grouped_fp32_shapes(gpu_lib, n, k, gs):
    if k % gs:
        pytest.skip("group does not divide k")
    w_vals, w_dev = weight_tensor(WL.normal(800 + k, (n, k), 0.02), "f32")
    grouped_roundtrip(gpu_lib, w_vals, w_dev, 0.73, gs)


@pytest.mark.parametrize("n,k,gs", [(1, 32, 32), (3, 96, 32), (5, 160, 32), (9, 192, 64)])
def test_grouped_ragged_flat_tails(gpu_lib, n, k, gs):
    """n*k not a multiple of the 1024 elements a wave takes per batch."""
    w_vals, w_dev = weight_tensor(WL.student_t(900 + n * k, (n, k)), "bf16")
    grouped_roundtrip(gpu_lib, w_vals, w_dev, 0.73, gs)


def _special_groups(gs):
    """One row, one special group after another (float32)."""
    rng = np.random.default_rng(17)
    groups = []
    groups.append(np.zeros(gs, np.float32))                                   # all zero
    g = np.zeros(gs, np.float32); g[::3] = -0.0; groups.append(g)             # signed zeros
    g = (rng.standard_normal(gs) * 2.0 ** -27).astype(np.float32); groups.append(g)  # max rounds to 0
    g = np.zeros(gs, np.float32); g[1] = 2.0 ** -25; g[2] = -(2.0 ** -26); groups.append(g)  # tie to 0
    g = (rng.standard_normal(gs) * 3e-7).astype(np.float32); groups.append(g)  # float16 subnormal max
    g = (rng.standard_normal(gs) * 0.02).astype(np.float32); g[3] = 1.0 + 2.0 ** -12
    g[4] = -(1.0 + 2.0 ** -13); groups.append(g)                               # max rounds down: u > 1
    g = (rng.standard_normal(gs) * 3e4).astype(np.float32); g[0] = 1e5; groups.append(g)  # saturates
    g = (rng.standard_normal(gs) * 0.02).astype(np.float32); g[7] = 0.1; groups.append(g)  # rounds up
    groups.append(np.full(gs, -0.25, np.float32))                              # constant magnitude
    groups.append(np.linspace(-1, 1, gs).astype(np.float32))
    return np.concatenate(groups)[None, :]


@pytest.mark.parametrize("gs", GROUPS)
@pytest.mark.parametrize("alpha", [0.1, 0.45, 0.73, 1.0, 2.0])
def test_grouped_special_groups(gpu_lib, gs, alpha):
    w = _special_groups(gs)
    pad = (-w.shape[1]) % 256
    w = np.concatenate([w, np.zeros((1, pad), np.float32)], axis=1)
    w = np.concatenate([w, -w[:, ::-1]], axis=0)
    for dtype in ("f32", "bf16"):
        w_vals, w_dev = weight_tensor(w, dtype)
        grouped_roundtrip(gpu_lib, w_vals, w_dev, alpha, gs)


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0])
def test_grouped_near_decision_points(gpu_lib, alpha):
    """Magnitudes within a few binary32 ulps of T_k * m16 in each group (the
    exact path of the encoder)."""
    gs = 64
    t = O.decision_thresholds_f32(alpha)
    groups = []
    for m16 in (np.float32(0.03711), np.float32(1.0), np.float32(0.0031)):
        m16 = np.float32(np.float16(m16))
        for tk in t:
            ci = int(np.array([tk * m16], np.float32).view(np.int32)[0])
            vals = np.arange(ci - 31, ci + 32, dtype=np.int32).view(np.float32)
            vals = vals[(vals >= 0) & (vals <= m16)][:gs - 1]
            g = np.zeros(gs, np.float32)
            g[:len(vals)] = vals
            g[gs - 1] = m16
            g *= np.where(np.arange(gs) % 2 == 1, -1.0, 1.0).astype(np.float32)
            groups.append(g)
    w = np.concatenate(groups)[None, :]
    w = np.concatenate([w, np.zeros((1, (-w.shape[1]) % 256), np.float32)], axis=1)
    w_vals, w_dev = weight_tensor(w, "f32")
    grouped_roundtrip(gpu_lib, w_vals, w_dev, alpha, gs)


@pytest.mark.parametrize("m,n,k,gs", [
    (1, 300, 512, 128), (8, 256, 256, 32), (16, 129, 96, 32), (32, 200, 768, 64),
    (33, 200, 768, 64), (64, 100, 1024, 256), (65, 96, 256, 128), (200, 300, 544, 32),
    (256, 512, 1024, 128), (300, 260, 3840, 256), (130, 64, 192, 64),
    # skinny blocks with 16 x k/gs group tables: one per thread of the block
    # (made at block start), and more (rebuilt per k block)
    (16, 50, 1024, 32), (40, 50, 8192, 256), (16, 50, 4096, 32), (8, 40, 8192, 128),
    (33, 24, 4160, 32)])
def test_grouped_linear_shapes(gpu_lib, m, n, k, gs):
    opq = gpu_lib
    w_vals, w_dev = weight_tensor(WL.student_t(1000 + n + gs, (n, k)), "bf16")
    gw = quantize_grouped_guarded(opq, w_dev, 0.73, gs)
    ref = O.quantize_grouped(w_vals, 0.73, gs)
    assert_grouped_equal(gw, ref)
    d_ref = O.dequantize_grouped(*ref, 0.73, gs)
    xt = to_bf16(WL.normal(1100 + m, (m, k)))
    bias = WL.normal(1200 + n, (n,), 0.5)
    gy = Guarded((m, n), torch.float32)
    opq.linear(xt.to(DEV), gw, 0.73, bias=torch.from_numpy(bias).to(DEV), out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    assert_linear_close(gy.t.cpu().numpy(), O.linear(bf16_bits(xt), d_ref, bias))
    # bf16 output: the float32 result rounded once more
    gb = Guarded((m, n), torch.bfloat16)
    opq.linear(xt.to(DEV), gw, 0.73, bias=torch.from_numpy(bias).to(DEV), out=gb.t)
    torch.cuda.synchronize()
    gb.check()
    y32 = gy.t.cpu().numpy()
    b = y32.view(np.uint32).astype(np.uint64)
    assert np.array_equal(bf16_bits(gb.t.cpu()), ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16))


def test_grouped_linear_one_hot_rows(gpu_lib):
    """x = identity rows: y[:, n] is the group-wise reconstruction W'[n, :]."""
    opq = gpu_lib
    k, n = 256, 96
    for gs in GROUPS:
        _, w_dev = weight_tensor(WL.student_t(1300 + gs, (n, k)), "bf16")
        gw = opq.quantize_grouped(w_dev, 0.73, gs)
        d = opq.dequantize(gw, 0.73)
        for m in (k, 64):
            x = torch.eye(k, dtype=torch.bfloat16, device=DEV)[:m].contiguous()
            y = opq.linear(x, gw, 0.73)
            assert torch.equal(y, d[:, :m].float().t().contiguous()), (gs, m)


def test_grouped_empty_calls(gpu_lib):
    opq = gpu_lib
    gw = opq.quantize_grouped(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), 0.73, 128)
    assert gw.scale16.shape == (0, 2)
    gw = opq.quantize_grouped(torch.empty((4, 0), dtype=torch.bfloat16, device=DEV), 0.73, 64)
    assert opq.dequantize(gw, 0.73).shape == (4, 0)
    bias = torch.arange(4, dtype=torch.float32, device=DEV)
    for m in (3, 100):
        y = opq.linear(torch.empty((m, 0), dtype=torch.bfloat16, device=DEV), gw, 0.73, bias=bias)
        assert torch.equal(y.cpu(), bias.cpu().expand(m, 4))


@pytest.mark.parametrize("key", ["skinny", "qkv"])
def test_grouped_full_size(gpu_lib, key):
    """The configs' weights at full size in groups of 128: every stored word
    against the oracle on sampled rows; the linear layer on sampled x rows."""
    opq = gpu_lib
    L = WL.config(key).layers[0]
    w32 = L.make_w()
    w_vals, w_dev = weight_tensor(w32, L.w_dtype)
    del w32
    gw = opq.quantize_grouped(w_dev, WL.ALPHA, 128)
    rng = np.random.default_rng(L.n)
    rows = np.unique(np.concatenate([[0, L.n - 1], rng.choice(L.n, 384, replace=False)]))
    ref = O.quantize_grouped(w_vals[rows], WL.ALPHA, 128)
    torch.cuda.synchronize()
    assert_grouped_equal(gw, ref, rows)
    d = opq.dequantize(gw, WL.ALPHA)
    assert np.array_equal(bf16_bits(d[torch.from_numpy(rows).to(DEV)]),
                          O.dequantize_grouped(*ref, WL.ALPHA, 128))
    del d
    full = O.quantize_grouped(w_vals, WL.ALPHA, 128)
    d_ref = O.dequantize_grouped(*full, WL.ALPHA, 128)
    xt = to_bf16(L.make_x())
    y = opq.linear(xt.to(DEV), gw, WL.ALPHA)
    xr = np.unique(np.concatenate([[0, L.m - 1], rng.choice(L.m, min(L.m, 48), replace=False)]))
    assert_linear_close(y[torch.from_numpy(xr).to(DEV)].cpu().numpy(),
                        O.linear(bf16_bits(xt)[xr], d_ref))
