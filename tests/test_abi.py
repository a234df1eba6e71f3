"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
and its host-only parts (tables, argument checks, empty calls) behave as
include/opq.h states.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import mpmath
import numpy as np
import pytest

import oracle as O
from w4a16_linear_amd import opq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "opq.h")

OK, NULL, SHAPE, ALPHA, ALIGN, DTYPE, WORKSPACE, UNSUPPORTED, HIP = range(9)
FAKE = 0x7F0000000000          # an aligned, never dereferenced address
MISALIGNED = FAKE + 4


@pytest.fixture(scope="module")
def lib():
    return opq.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(opq_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 18
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(opq._SIGNATURES)


def test_abi_version_and_status_text(lib):
    assert lib.opq_abi_version() == opq.ABI_VERSION == 6
    for s in range(9):
        assert opq.status_str(s) and opq.status_str(s) != "unknown status"
    assert opq.status_str(99) == "unknown status"


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0, 0.5, 0.25, 2.0, 0.3, 3.7, 0.05, 10.0, 0.999])
def test_decision_points_equal_oracle(alpha):
    """The library's binary128 search and the oracle's mpmath search agree."""
    got = opq.decision_points(alpha)
    ref = O.decision_thresholds_f32(alpha)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("alpha", [0.45, 0.73, 1.0, 2.5])
def test_levels(alpha):
    g = opq.levels(alpha)
    assert g[0] == 0.0 and g[15] == 1.0
    a = mpmath.mpf(O.alpha_f32(alpha))
    with mpmath.workprec(120):
        for q in range(1, 15):
            ex = mpmath.power(mpmath.mpf(q) / 15, 1 / a)
            assert abs(g[q] - float(ex)) <= np.spacing(float(ex))  # rounded from binary128


def test_table_argument_errors(lib):
    buf = np.zeros(16, np.float64)
    assert lib.opq_decision_points(0.73, None) == NULL
    assert lib.opq_levels(0.73, None) == NULL
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.opq_decision_points(bad, buf.ctypes.data) == ALPHA
        assert lib.opq_levels(bad, buf.ctypes.data) == ALPHA


def test_quantize_argument_checks(lib):
    q = lib.opq_quantize
    assert q(None, 1, 4, 64, 0.73, FAKE, FAKE, FAKE, None) == NULL
    assert q(FAKE, 1, 4, 64, 0.73, FAKE, None, FAKE, None) == NULL
    assert q(None, 1, 4, 63, 0.0, FAKE, FAKE, FAKE, None) == NULL      # null first
    assert q(FAKE, 1, 4, 48, 0.73, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 1, -1, 64, 0.73, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 1, 4, -32, 0.73, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 1, 4, 48, -1.0, FAKE, FAKE, FAKE, None) == SHAPE     # shape before alpha
    for bad in (0.0, -0.5, float("nan"), float("inf")):
        assert q(FAKE, 1, 4, 64, bad, FAKE, FAKE, FAKE, None) == ALPHA
    assert q(FAKE, 1, 4, 64, 0.0, MISALIGNED, FAKE, FAKE, None) == ALPHA
    assert q(MISALIGNED, 1, 4, 64, 0.73, FAKE, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 1, 4, 64, 0.73, FAKE, MISALIGNED, FAKE, None) == ALIGN
    assert q(FAKE, 1, 4, 64, 0.73, FAKE, FAKE, MISALIGNED, None) == ALIGN
    assert q(FAKE, 7, 4, 64, 0.73, MISALIGNED, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 7, 4, 64, 0.73, FAKE, FAKE, FAKE, None) == DTYPE
    assert q(FAKE, 1, 4, 65536 + 32, 0.73, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, 1, 0, 64, 0.73, FAKE, FAKE, FAKE, None) == OK         # empty: nothing enqueued


def test_error_sums_argument_checks(lib):
    e = lib.opq_error_sums
    assert e(None, 1, 4, 64, 0.73, FAKE, None) == NULL
    assert e(FAKE, 1, 4, 64, 0.73, None, None) == NULL
    assert e(FAKE, 1, 4, 40, 0.73, FAKE, None) == SHAPE
    assert e(FAKE, 1, 4, 64, -1.0, FAKE, None) == ALPHA
    assert e(FAKE, 1, 4, 64, 0.73, MISALIGNED, None) == ALIGN
    assert e(FAKE, 5, 4, 64, 0.73, FAKE, None) == DTYPE
    assert e(FAKE, 1, 4, 16384 + 32, 0.73, FAKE, None) == UNSUPPORTED
    assert e(FAKE, 1, 4, 64, 100.0, FAKE, None) == UNSUPPORTED  # no separating bucket grid
    assert e(FAKE, 1, 4, 64, 0.03, FAKE, None) == UNSUPPORTED   # nor here (T_1 below 2^-126)
    assert e(FAKE, 1, 0, 64, 0.73, FAKE, None) == OK           # empty: nothing enqueued


def test_dequantize_argument_checks(lib):
    d = lib.opq_dequantize
    assert d(FAKE, None, FAKE, 4, 64, 0.73, FAKE, None) == NULL
    assert d(FAKE, FAKE, FAKE, 4, 40, 0.73, FAKE, None) == SHAPE
    assert d(FAKE, FAKE, FAKE, 4, 64, float("nan"), FAKE, None) == ALPHA
    assert d(FAKE, FAKE, FAKE, 4, 64, 0.73, MISALIGNED, None) == ALIGN
    assert d(FAKE, FAKE, FAKE, 0, 64, 0.73, FAKE, None) == OK
    assert d(FAKE, FAKE, FAKE, 4, 0, 0.73, FAKE, None) == OK


def test_linear_argument_checks(lib):
    f = lib.opq_linear
    args = dict(x=FAKE, p=FAKE, s=FAKE, sc=FAKE, b=None, m=8, n=16, k=64, a=0.73, y=FAKE,
                yd=0, ws=None, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["p"], a["s"], a["sc"], a["b"], a["m"], a["n"], a["k"], a["a"], a["y"],
                 a["yd"], a["ws"], a["wsb"], None)

    assert call(x=None) == NULL
    assert call(y=None) == NULL
    assert call(k=33) == SHAPE
    assert call(m=-1) == SHAPE
    assert call(a=0.0) == ALPHA
    assert call(b=MISALIGNED) == ALIGN
    assert call(x=MISALIGNED) == ALIGN
    assert call(ws=MISALIGNED) == ALIGN
    assert call(yd=7) == DTYPE
    assert call(yd=7, y=MISALIGNED) == ALIGN          # alignment is checked before dtype
    assert call(m=0) == OK
    assert call(n=0) == OK
    assert call(m=0, yd=1) == OK
    assert call(k=65536 + 32) == UNSUPPORTED
    assert call(n=(1 << 26) + 1) == UNSUPPORTED   # past the skinny kernel's 32-bit grid
    assert lib.opq_linear_workspace_bytes(8, 16, 64) == opq.linear_workspace_bytes(8, 16, 64)


def test_bits_argument_checks(lib):
    q = lib.opq_quantize_bits
    assert q(None, 1, 4, 64, 3, 0.73, FAKE, FAKE, FAKE, None) == NULL
    for b in (0, 1, 2, 7, 8, -4):
        assert q(FAKE, 1, 4, 64, b, 0.73, FAKE, FAKE, FAKE, None) == SHAPE, b
    assert q(FAKE, 1, 4, 48, 5, 0.73, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 1, 4, 64, 6, 0.0, FAKE, FAKE, FAKE, None) == ALPHA
    assert q(FAKE, 1, 4, 64, 6, 0.73, MISALIGNED, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 4, 4, 64, 6, 0.73, FAKE, FAKE, FAKE, None) == DTYPE
    assert q(FAKE, 1, 4, 16384 + 32, 6, 0.73, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, 1, 4, 64, 6, 100.0, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, 1, 0, 64, 3, 0.73, FAKE, FAKE, FAKE, None) == OK
    # bits = 4 is opq_quantize itself (same checks, its own k limit)
    assert q(FAKE, 1, 4, 65536 + 32, 4, 0.73, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    d = lib.opq_dequantize_bits
    assert d(FAKE, None, FAKE, 4, 64, 5, 0.73, FAKE, None) == NULL
    assert d(FAKE, FAKE, FAKE, 4, 64, 9, 0.73, FAKE, None) == SHAPE
    assert d(FAKE, FAKE, FAKE, 4, 64, 5, -1.0, FAKE, None) == ALPHA
    assert d(FAKE, FAKE, FAKE, 4, 64, 5, 0.73, MISALIGNED, None) == ALIGN
    assert d(FAKE, FAKE, FAKE, 4, 65536 + 32, 5, 0.73, FAKE, None) == UNSUPPORTED
    assert d(FAKE, FAKE, FAKE, 0, 64, 5, 0.73, FAKE, None) == OK
    e = lib.opq_error_sums_bits
    assert e(FAKE, 1, 4, 64, 3, 0.73, None, None) == NULL
    assert e(FAKE, 1, 4, 64, 2, 0.73, FAKE, None) == SHAPE
    assert e(FAKE, 1, 4, 16384 + 32, 5, 0.73, FAKE, None) == UNSUPPORTED
    assert e(FAKE, 1, 0, 64, 6, 0.73, FAKE, None) == OK


def test_linear_bits_argument_checks(lib):
    f = lib.opq_linear_bits
    ws_need = lib.opq_linear_bits_workspace_bytes(8, 16, 64, 5)
    args = dict(x=FAKE, p=FAKE, s=FAKE, sc=FAKE, b=None, m=8, n=16, k=64, bits=5, a=0.73, y=FAKE,
                yd=0, ws=FAKE, wsb=ws_need)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["p"], a["s"], a["sc"], a["b"], a["m"], a["n"], a["k"], a["bits"],
                 a["a"], a["y"], a["yd"], a["ws"], a["wsb"], None)

    assert ws_need == 16 * 64 * 2                    # W' as bfloat16, already a multiple of 256
    assert lib.opq_linear_bits_workspace_bytes(8, 3, 32, 3) == 256   # 192 bytes rounded up
    assert lib.opq_linear_bits_workspace_bytes(0, 16, 64, 6) == 0
    assert lib.opq_linear_bits_workspace_bytes(8, 16, 64, 4) == lib.opq_linear_workspace_bytes(8, 16, 64)
    assert call(x=None) == NULL
    assert call(sc=None) == NULL
    assert call(k=48) == SHAPE
    for b in (2, 7, 0):
        assert call(bits=b) == SHAPE, b
    assert call(a=float("nan")) == ALPHA
    assert call(ws=MISALIGNED) == ALIGN
    assert call(yd=3) == DTYPE
    assert call(wsb=ws_need - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(m=0, ws=None, wsb=0) == OK
    assert call(n=0, ws=None, wsb=0) == OK
    assert call(k=65536 + 32, wsb=16 * (65536 + 32) * 2) == UNSUPPORTED
    # bits = 4 is opq_linear itself (no workspace needed)
    assert call(bits=4, ws=None, wsb=0, k=65536 + 32) == UNSUPPORTED
    assert call(bits=4, ws=None, wsb=0, m=0) == OK


def test_linear_bits_noalloc_argument_checks(lib):
    """The allocation-free variant checks like opq_linear_bits and refuses
    shapes whose W' exceeds its fixed 160 MiB (without enqueuing anything)."""
    f = lib.opq_linear_bits_noalloc

    def call(x=FAKE, sc=FAKE, m=8, n=16, k=64, bits=5, a=0.73, y=FAKE, yd=0):
        return f(x, FAKE, FAKE, sc, None, m, n, k, bits, a, y, yd, None)

    assert call(x=None) == NULL
    assert call(bits=7) == SHAPE
    assert call(a=-1.0) == ALPHA
    assert call(y=MISALIGNED) == ALIGN
    assert call(yd=9) == DTYPE
    assert call(m=0) == OK and call(n=0) == OK
    big_n = (160 << 20) // (2 * 4096) + 1              # n * 4096 * 2 bytes just past 160 MiB
    assert call(n=big_n, k=4096) == UNSUPPORTED
    assert call(n=big_n, k=4096, x=None) == NULL        # argument errors keep their codes
    assert call(n=big_n - 1, k=4096, m=0) == OK
    assert call(bits=4, k=65536 + 32) == UNSUPPORTED    # opq_linear's own limit


def test_grouped_argument_checks(lib):
    q = lib.opq_quantize_grouped
    assert q(None, 1, 4, 256, 128, 0.73, FAKE, FAKE, FAKE, None) == NULL
    assert q(FAKE, 1, 4, 256, 128, 0.73, FAKE, FAKE, None, None) == NULL
    for gs in (16, 48, 100, 512, 0, -32):
        assert q(FAKE, 1, 4, 512, gs, 0.73, FAKE, FAKE, FAKE, None) == SHAPE, gs
    assert q(FAKE, 1, 4, 96, 64, 0.73, FAKE, FAKE, FAKE, None) == SHAPE   # 64 does not divide 96
    assert q(FAKE, 1, 4, 96, 64, 0.0, FAKE, FAKE, FAKE, None) == SHAPE    # shape before alpha
    assert q(FAKE, 1, 4, 256, 128, -1.0, FAKE, FAKE, FAKE, None) == ALPHA
    assert q(FAKE, 1, 4, 256, 128, 0.73, FAKE, FAKE, MISALIGNED, None) == ALIGN
    assert q(FAKE, 3, 4, 256, 128, 0.73, FAKE, FAKE, FAKE, None) == DTYPE
    assert q(FAKE, 1, 4, 256, 128, 100.0, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, 1, 4, 256, 128, 0.03, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert q(FAKE, 1, 0, 256, 128, 0.73, FAKE, FAKE, FAKE, None) == OK
    assert q(FAKE, 1, 4, 0, 128, 0.73, FAKE, FAKE, FAKE, None) == OK
    d = lib.opq_dequantize_grouped
    assert d(FAKE, FAKE, None, 4, 256, 128, 0.73, FAKE, None) == NULL
    assert d(FAKE, FAKE, FAKE, 4, 256, 96, 0.73, FAKE, None) == SHAPE
    assert d(FAKE, FAKE, FAKE, 4, 256, 128, float("inf"), FAKE, None) == ALPHA
    assert d(FAKE, FAKE, MISALIGNED, 4, 256, 128, 0.73, FAKE, None) == ALIGN
    assert d(FAKE, FAKE, FAKE, 4, 256, 128, 100.0, FAKE, None) == UNSUPPORTED
    assert d(FAKE, FAKE, FAKE, 0, 256, 128, 0.73, FAKE, None) == OK
    f = lib.opq_linear_grouped
    args = dict(x=FAKE, p=FAKE, s=FAKE, sc=FAKE, b=None, m=8, n=16, k=256, gs=128, a=0.73, y=FAKE,
                yd=0, ws=None, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["p"], a["s"], a["sc"], a["b"], a["m"], a["n"], a["k"], a["gs"], a["a"],
                 a["y"], a["yd"], a["ws"], a["wsb"], None)

    assert call(sc=None) == NULL
    assert call(gs=512) == SHAPE
    assert call(k=320, gs=256) == SHAPE
    assert call(a=-2.0) == ALPHA
    assert call(sc=MISALIGNED) == ALIGN
    assert call(yd=2) == DTYPE
    assert call(a=100.0) == UNSUPPORTED
    assert call(k=65536 + 256, gs=256) == UNSUPPORTED
    assert call(n=(1 << 26) + 1) == UNSUPPORTED
    assert call(m=0) == OK and call(n=0) == OK


def test_linear_workspace_sizes(lib):
    """Only the split-k tiled layer keeps partial sums: few 256 x 256 tiles
    with k a multiple of 64.  Skinny, large-m, invalid and empty shapes need
    none."""
    ws = lib.opq_linear_workspace_bytes
    for m, n, k in [(1, 3840, 3840), (32, 3840, 3840), (64, 3840, 10240), (4096, 11520, 3840),
                    (4096, 20480, 3840), (4096, 3840, 10240), (0, 3840, 3840), (32, 0, 3840),
                    (-1, 3840, 3840), (32, 3840, 65536 + 32), (32, 3840, 100),
                    (1024, 3840, 3840 + 32), (200, 300, 544), (65, 3840, 3840), (128, 3840, 3840),
                    (2048, 3840, 3840)]:
        assert ws(m, n, k) == 0, (m, n, k)
    for m, n, k in [(1024, 3840, 3840), (256, 3840, 3840), (512, 1024, 8192), (130, 1024, 8192)]:
        b = ws(m, n, k)
        assert b % 256 == 0 and 2 * m * n * 4 <= b <= 128 << 20, (m, n, k, b)
    # 60 tiles: 4 slices of 16, 16, 16 and 12 k steps
    assert ws(1024, 3840, 3840) == 4 * 1024 * 3840 * 4


def test_linear_workspace_checked(lib):
    f = lib.opq_linear
    need = lib.opq_linear_workspace_bytes(1024, 3840, 3840)

    def call(ws, wsb):
        return f(FAKE, FAKE, FAKE, FAKE, None, 1024, 3840, 3840, 0.73, FAKE, 0, ws, wsb, None)

    assert call(None, 0) == WORKSPACE
    assert call(FAKE, need - 1) == WORKSPACE
    assert call(None, need) == WORKSPACE


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        opq.quantize(torch.zeros(4, 64), 0.73)
    with pytest.raises(ValueError):
        opq.quantize(torch.zeros(4, 64, dtype=torch.float16), 0.73)


def test_host_tables_are_thread_safe():
    """Many threads asking for many alphas at once (the per-alpha memo is the
    library's only global state): every answer equals the single-threaded one."""
    import threading
    alphas = [0.3 + 0.05 * i for i in range(20)]
    want = {a: opq.decision_points(a).tobytes() + opq.levels(a).tobytes() for a in alphas}
    bad = []

    def worker(seed):
        rng = np.random.default_rng(seed)
        for a in rng.choice(alphas, 200):
            got = opq.decision_points(a).tobytes() + opq.levels(a).tobytes()
            if got != want[a]:
                bad.append(a)

    threads = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad


def test_ceiling_library_checks_arguments():
    """The benchmark's streaming-ceiling library loads and refuses bad
    arguments before any launch (no GPU needed for these)."""
    import ctypes
    from w4a16_linear_amd import build as B
    lib = ctypes.CDLL(B.CEILING_LIB)
    f = lib.opq_ceiling_stream_rows
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p]
    assert f(FAKE, FAKE, 0, 16, 16, None) == 0           # nothing to do
    assert f(FAKE, FAKE, 4, 24, 16, None) == 1           # not a multiple of 16
    assert f(FAKE, FAKE, -1, 16, 16, None) == 1
    assert f(None, FAKE, 4, 16, 16, None) == 1
    assert f(FAKE, None, 4, 16, 16, None) == 1
    assert f(MISALIGNED, FAKE, 4, 16, 16, None) == 1
    assert f(FAKE, FAKE, 4, 1 << 31, 16, None) == 1
