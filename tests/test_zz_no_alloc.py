"""The allocation-free b-bit linear layer (opq_linear_bits_noalloc) against
opq_linear_bits with a caller workspace, through the C ABI: two calls in a row
on the library's fixed per-GPU scratch, the second smaller, each equal bit for
bit to the workspace call (the same kernels on the same W'), and both within
the linear tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from w4a16_linear_amd import workloads as WL
from w4a16_linear_amd.workloads import bf16_bits, u32

from test_gpu_parity import DEV, Guarded, assert_linear_close, weight_tensor

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 160 << 20


def _case(opq, m, n, k, bits, alpha, seed, bias=False):
    print(f"noalloc case: bits={bits} m={m} n={n} k={k} alpha={alpha} seed={seed}", flush=True)
    w_vals, w_dev = weight_tensor(WL.student_t(seed, (n, k)), "bf16")
    bw = opq.quantize_bits(w_dev, alpha, bits)
    xt = WL.to_bf16(WL.normal(seed + 1, (m, k)))
    x = xt.to(DEV)
    b = torch.from_numpy(WL.normal(seed + 2, (n,), 0.1)) if bias else None
    bd = None if b is None else b.to(DEV)
    ws = torch.empty(max(opq.linear_workspace_bytes(m, n, k, bits), 1), dtype=torch.uint8,
                     device=DEV)
    y_ws = opq.linear(x, bw, alpha, bias=bd, workspace=ws)
    gy = Guarded((m, n), torch.float32)
    opq.linear_noalloc(x, bw, alpha, bias=bd, out=gy.t)
    torch.cuda.synchronize()
    gy.check()
    assert torch.equal(gy.t, y_ws), "noalloc output differs from the workspace call"
    p_ref, s_ref, m_ref = O.quantize_bits(w_vals, alpha, bits)
    assert np.array_equal(u32(bw.packed), p_ref) and np.array_equal(u32(bw.sign), s_ref)
    d_ref = O.dequantize_bits(p_ref, s_ref, m_ref, alpha, bits)
    y_ref = O.linear(bf16_bits(xt), d_ref, None if b is None else b.numpy())
    return assert_linear_close(gy.t.cpu().numpy(), y_ref)


def test_noalloc_two_calls_second_smaller(gpu_lib):
    """A tiled call (m > 64, ragged n and k) fills much of the scratch; a
    smaller skinny call with other bits then reuses it."""
    _case(gpu_lib, 300, 2000, 3872, 5, 0.73, 2600, bias=True)
    _case(gpu_lib, 20, 256, 512, 3, 0.45, 2610)


def test_noalloc_each_width_and_4bit(gpu_lib):
    """Widths 6 and 4, larger then smaller.  Width 4 is opq_linear: 300 x 1000 x
    4096 splits k over the tiles and keeps its partial sums in the scratch,
    200 x 640 x 1024 and 8 x 96 x 256 need none."""
    assert gpu_lib.linear_workspace_bytes(300, 1000, 4096) > 0
    assert gpu_lib.linear_workspace_bytes(200, 640, 1024) == 0
    for bits, m, n, k in ((6, 130, 1500, 2048), (6, 33, 100, 160), (4, 300, 1000, 4096),
                          (4, 200, 640, 1024), (4, 8, 96, 256)):
        _case(gpu_lib, m, n, k, bits, 1.0, 2620 + bits + m)


def test_noalloc_largest_fitting_layer(gpu_lib):
    """The FFN up/gate projection (W' of 20480 x 3840 bfloat16, 150 MiB) fits;
    one row more than the scratch holds is refused before any launch."""
    opq = gpu_lib
    n, k, m, bits = 20480, 3840, 64, 5
    assert n * k * 2 <= SCRATCH_BYTES
    _, w_dev = weight_tensor(WL.student_t(2700, (n, k)), "bf16")
    bw = opq.quantize_bits(w_dev, 0.73, bits)
    x = WL.to_bf16(WL.normal(2701, (m, k))).to(DEV)
    y_ws = opq.linear(x, bw, 0.73)
    y = opq.linear_noalloc(x, bw, 0.73)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ws)
    n_big = SCRATCH_BYTES // (2 * k) + 1
    big = opq.BitsWeight(torch.zeros((n_big, k * bits // 32), dtype=torch.int32, device=DEV),
                         torch.zeros((n_big, k // 32), dtype=torch.int32, device=DEV),
                         torch.ones((n_big,), dtype=torch.float32, device=DEV), bits)
    with pytest.raises(opq.OpqError) as e:
        opq.linear_noalloc(x, big, 0.73)
    assert e.value.status == 7   # OPQ_ERR_UNSUPPORTED
    # the refusal left the scratch usable
    x7 = x[:7].contiguous()
    y2 = opq.linear_noalloc(x7, bw, 0.73)
    y2_ws = opq.linear(x7, bw, 0.73)
    torch.cuda.synchronize()
    assert torch.equal(y2, y2_ws)
