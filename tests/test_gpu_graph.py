"""The library's calls under HIP graph capture: quantize, dequantize and the
linear layer (per-row and group-wise, skinny and tiled, and the tiled layer
with k split over a workspace and a second, reducing kernel) captured once in a
torch CUDA graph and replayed several times, with eager work and
synchronisations between the replays; every replay's outputs equal the eager
call's bit for bit (the calls enqueue kernels only, no memset or copy)."""
import pytest
import torch

from w4a16_linear_amd import workloads as WL

from test_gpu_parity import DEV, weight_tensor

pytestmark = pytest.mark.gpu

ALPHA = 0.73


def _eager(opq, w, x_small, x_big, x_split, group):
    if group:
        qw = opq.quantize_grouped(w, ALPHA, group)
    else:
        qw = opq.quantize(w, ALPHA)
    d = opq.dequantize(qw, ALPHA)
    ys = opq.linear(x_small, qw, ALPHA)
    yb = opq.linear(x_big, qw, ALPHA)
    yk = opq.linear(x_split, qw, ALPHA)
    torch.cuda.synchronize()
    return qw, d, ys, yb, yk


@pytest.mark.parametrize("group", [0, 128])
def test_graph_replays_match_eager(gpu_lib, group):
    opq = gpu_lib
    n, k = 384, 1024
    _, w = weight_tensor(WL.student_t(2100 + group, (n, k)), "bf16")
    x_small = WL.to_bf16(WL.normal(2200, (16, k))).to(DEV)
    x_big = WL.to_bf16(WL.normal(2201, (300, k))).to(DEV)
    x_split = WL.to_bf16(WL.normal(2202, (1024, k))).to(DEV)
    if not group:  # per-row scales: the 1024-row call splits k
        assert opq.linear_workspace_bytes(1024, n, k) > 0
    qw_ref, d_ref, ys_ref, yb_ref, yk_ref = _eager(opq, w, x_small, x_big, x_split, group)

    # static outputs the captured calls write into
    if group:
        qw = opq.GroupedWeight(torch.empty_like(qw_ref.packed), torch.empty_like(qw_ref.sign),
                               torch.empty_like(qw_ref.scale16), group)
    else:
        qw = opq.QuantizedWeight(torch.empty_like(qw_ref.packed), torch.empty_like(qw_ref.sign),
                                 torch.empty_like(qw_ref.scale))
    d = torch.empty_like(d_ref)
    ys = torch.empty_like(ys_ref)
    yb = torch.empty_like(yb_ref)
    yk = torch.empty_like(yk_ref)

    def calls():
        if group:
            opq.quantize_grouped(w, ALPHA, group, out=qw)
        else:
            opq.quantize(w, ALPHA, out=qw)
        opq.dequantize(qw, ALPHA, out=d)
        opq.linear(x_small, qw, ALPHA, out=ys)
        opq.linear(x_big, qw, ALPHA, out=yb)
        opq.linear(x_split, qw, ALPHA, out=yk)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()  # warm the binding's caches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (qw.packed, qw.sign, d, ys, yb, yk):
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qw.packed, qw_ref.packed), rep
        assert torch.equal(qw.sign, qw_ref.sign), rep
        if group:
            assert torch.equal(qw.scale16, qw_ref.scale16), rep
        else:
            assert torch.equal(qw.scale, qw_ref.scale), rep
        assert torch.equal(d, d_ref), rep
        assert torch.equal(ys, ys_ref), rep
        assert torch.equal(yb, yb_ref), rep
        assert torch.equal(yk, yk_ref), rep
