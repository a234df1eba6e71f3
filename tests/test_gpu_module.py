"""The torch front end on the GPU against the oracle: replace_with_opq stores
the oracle's codes bit for bit, each OPQLinear's output meets the linear
tolerance against the oracle's product on the inputs that layer saw, and a
save / load round trip reproduces the outputs bit for bit."""
import math

import numpy as np
import pytest
import torch
from torch import nn

import oracle as O
from w4a16_linear_amd import workloads as WL
from w4a16_linear_amd.module import OPQLinear, load_opq, replace_with_opq, save_opq
from w4a16_linear_amd.workloads import bf16_bits

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LINEAR_TOL = 1e-2


def _stack(dtype, seed):
    """A small synthetic stack: in 256 -> 512 -> 384 -> 128 (last layer without
    bias), GELU between, Student-t(4) weights at std 0.02."""
    model = nn.Sequential(nn.Linear(256, 512), nn.GELU(), nn.Linear(512, 384), nn.GELU(),
                          nn.Linear(384, 128, bias=False))
    with torch.no_grad():
        for i, lin in enumerate(m for m in model if isinstance(m, nn.Linear)):
            n, k = lin.weight.shape
            lin.weight.copy_(torch.from_numpy(WL.student_t(seed + i, (n, k))))
            if lin.bias is not None:
                lin.bias.copy_(torch.from_numpy(WL.normal(seed + 10 + i, (n,), 0.1)))
    return model.to(device=DEV, dtype=dtype)


def _bf16_rne_bits(y32):
    b = y32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _check_layer_output(x_in, y_out, ref_w_bits, bias):
    """y_out (the layer's output for input x_in) against the oracle's product."""
    x2 = x_in.reshape(-1, x_in.shape[-1]).to(torch.bfloat16)
    y_ref = O.linear(bf16_bits(x2.cpu()), ref_w_bits,
                     None if bias is None else bias.detach().float().cpu().numpy())
    y = y_out.reshape(-1, y_out.shape[-1]).float().cpu().numpy().astype(np.float64)
    rms = math.sqrt(float(np.mean(y_ref * y_ref)))
    # bf16 outputs: the float32 result rounded once more (half an ulp of y)
    half_ulp = 0.0
    if y_out.dtype == torch.bfloat16:
        yb = _bf16_rne_bits(y_ref.astype(np.float32)).astype(np.uint32) << 16
        half_ulp = np.abs(yb.view(np.float32).astype(np.float64) - y_ref)
    err = np.abs(y - y_ref) - half_ulp
    assert float(np.max(err)) <= LINEAR_TOL * rms, f"max err {np.max(err):.3e}, rms {rms:.3e}"


@pytest.mark.parametrize("dtype,alpha", [(torch.bfloat16, 0.73), (torch.float32, 0.45)])
def test_replace_with_opq_matches_oracle(gpu_lib, dtype, alpha):
    model = _stack(dtype, 7100)
    weights = {}
    for name, mod in model.named_modules():
        if isinstance(mod, nn.Linear):
            w = mod.weight.detach().float().cpu().numpy()
            weights[name] = (w, mod.bias)
    names = replace_with_opq(model, bits=4, alpha=alpha)
    assert names == ["0", "2", "4"]
    seen = {}
    hooks = [mod.register_forward_hook(lambda m, i, o, nm=name: seen.__setitem__(nm, (i[0], o)))
             for name, mod in model.named_modules() if isinstance(mod, OPQLinear)]
    for shape in ((4, 16, 256), (1, 256), (2, 100, 256)):   # m = 64, 1 (skinny), 200 (tiled)
        x = torch.from_numpy(WL.normal(7200 + shape[0], shape)).to(DEV, dtype)
        y = model(x)
        assert y.dtype == dtype and y.shape == shape[:-1] + (128,)
        for name, (w, bias) in weights.items():
            layer = model.get_submodule(name)
            ref = O.quantize(w, alpha)
            assert np.array_equal(layer.packed.cpu().numpy().view(np.uint32), ref[0])
            assert np.array_equal(layer.sign_packed.cpu().numpy().view(np.uint32), ref[1])
            assert np.array_equal(layer.mx.cpu().numpy().view(np.uint32), ref[2].view(np.uint32))
            d_ref = O.dequantize(*ref, alpha)
            assert np.array_equal(bf16_bits(layer.dequantized_weight().cpu()), d_ref)
            x_in, y_out = seen[name]
            _check_layer_output(x_in, y_out, d_ref, bias)
    for h in hooks:
        h.remove()


def test_save_load_reproduces_outputs(gpu_lib, tmp_path):
    model = _stack(torch.bfloat16, 7300)
    replace_with_opq(model, alpha=0.73)
    x = torch.from_numpy(WL.normal(7301, (3, 40, 256))).to(DEV, torch.bfloat16)
    y0 = model(x)
    path = str(tmp_path / "stack.safetensors")
    assert save_opq(model, path) == ["0", "2", "4"]
    fresh = _stack(torch.bfloat16, 9999)     # same structure, other weights
    assert load_opq(fresh, path) == ["0", "2", "4"]
    assert all(isinstance(fresh[i], OPQLinear) for i in (0, 2, 4))
    y1 = fresh(x)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def test_shared_linear_is_quantized_once(gpu_lib):
    lin = nn.Linear(64, 64).to(DEV)
    model = nn.Sequential(lin, nn.ReLU(), lin)
    assert replace_with_opq(model) == ["0", "2"]
    assert model[0] is model[2] and isinstance(model[0], OPQLinear)


def test_shared_layer_save_load(gpu_lib, tmp_path):
    lin = nn.Linear(64, 64).to(DEV)
    model = nn.Sequential(lin, nn.ReLU(), lin)
    replace_with_opq(model)
    path = str(tmp_path / "shared.safetensors")
    assert save_opq(model, path) == ["0"]
    skel_lin = nn.Linear(64, 64).to(DEV)
    skel = nn.Sequential(skel_lin, nn.ReLU(), skel_lin)
    load_opq(skel, path)
    assert skel[0] is skel[2] and isinstance(skel[0], OPQLinear)
    x = torch.from_numpy(WL.normal(7400, (5, 64))).to(DEV)
    assert torch.equal(model(x), skel(x))


@pytest.mark.parametrize("gs", [32, 128])
def test_grouped_layers_match_oracle_and_reload(gpu_lib, gs, tmp_path):
    model = _stack(torch.bfloat16, 7500)
    ws = {name: (mod.weight.detach().float().cpu().numpy(), mod.bias)
          for name, mod in model.named_modules() if isinstance(mod, nn.Linear)}
    assert replace_with_opq(model, alpha=0.73, group_size=gs) == ["0", "2", "4"]
    seen = {}
    for name, mod in model.named_modules():
        if isinstance(mod, OPQLinear):
            mod.register_forward_hook(lambda m, i, o, nm=name: seen.__setitem__(nm, (i[0], o)))
    x = torch.from_numpy(WL.normal(7501, (3, 30, 256))).to(DEV, torch.bfloat16)
    y0 = model(x)
    for name, (w, bias) in ws.items():
        layer = model.get_submodule(name)
        ref = O.quantize_grouped(w, 0.73, gs)
        assert np.array_equal(layer.packed.cpu().numpy().view(np.uint32), ref[0])
        assert np.array_equal(layer.mx.cpu().numpy().view(np.uint16), ref[2].view(np.uint16))
        d_ref = O.dequantize_grouped(*ref, 0.73, gs)
        assert np.array_equal(bf16_bits(layer.dequantized_weight().cpu()), d_ref)
        _check_layer_output(*seen[name], d_ref, bias)
    path = str(tmp_path / "grouped.safetensors")
    save_opq(model, path)
    fresh = _stack(torch.bfloat16, 1)
    load_opq(fresh, path)
    assert fresh[0].group_size == gs
    assert torch.equal(y0.view(torch.int16), fresh(x).view(torch.int16))


@pytest.mark.parametrize("bits", [3, 5, 6])
def test_bits_layers_match_oracle_and_reload(gpu_lib, bits, tmp_path):
    """replace_with_opq(bits=3|5|6): codes equal the oracle's b-bit codes, each
    layer's output meets the linear bar against the oracle's reconstruction
    (inputs of 3 x 30 and 100 x 1 tokens: the skinny and the tiled product),
    and a save / load round trip reproduces the outputs bit for bit."""
    model = _stack(torch.bfloat16, 7600 + bits)
    ws = {name: (mod.weight.detach().float().cpu().numpy(), mod.bias)
          for name, mod in model.named_modules() if isinstance(mod, nn.Linear)}
    assert replace_with_opq(model, bits=bits, alpha=0.73) == ["0", "2", "4"]
    seen = {}
    for name, mod in model.named_modules():
        if isinstance(mod, OPQLinear):
            assert mod.bits == bits
            mod.register_forward_hook(lambda m, i, o, nm=name: seen.__setitem__(nm, (i[0], o)))
    refs = {}
    for name, (w, bias) in ws.items():
        layer = model.get_submodule(name)
        ref = O.quantize_bits(w, 0.73, bits)
        assert np.array_equal(layer.packed.cpu().numpy().view(np.uint32), ref[0])
        assert np.array_equal(layer.sign_packed.cpu().numpy().view(np.uint32), ref[1])
        refs[name] = O.dequantize_bits(*ref, 0.73, bits)
    for shape in ((3, 30, 256), (100, 256)):
        x = torch.from_numpy(WL.normal(7601 + len(shape), shape)).to(DEV, torch.bfloat16)
        y0 = model(x)
        for name, (_, bias) in ws.items():
            _check_layer_output(*seen[name], refs[name], bias)
    path = str(tmp_path / "bits.safetensors")
    save_opq(model, path)
    fresh = _stack(torch.bfloat16, 1)
    load_opq(fresh, path)
    assert fresh[0].bits == bits
    assert torch.equal(y0.view(torch.int16), fresh(x).view(torch.int16))
