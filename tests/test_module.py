"""Host-side checks of the torch front end (OPQLinear, replace_with_opq,
save_opq / load_opq): structure, argument checks, the safetensors round trip
of the stored form, and that nothing computes off the GPU."""
import json

import numpy as np
import pytest
import torch
from torch import nn

from w4a16_linear_amd.module import FORMAT, OPQLinear, load_opq, replace_with_opq, save_opq


def _filled(in_f, out_f, bias, alpha, seed):
    g = torch.Generator().manual_seed(seed)
    m = OPQLinear(in_f, out_f, bias=bias, alpha=alpha)
    m.packed.copy_(torch.randint(-2**31, 2**31 - 1, m.packed.shape, dtype=torch.int32, generator=g))
    m.sign_packed.copy_(torch.randint(-2**31, 2**31 - 1, m.sign_packed.shape, dtype=torch.int32,
                                      generator=g))
    m.mx.copy_(torch.rand(out_f, generator=g))
    if bias:
        m.bias.copy_(torch.randn(out_f, generator=g))
    return m


def test_buffers_follow_the_stored_form():
    m = OPQLinear(96, 40, bias=True, alpha=0.73)
    assert m.packed.shape == (40, 12) and m.packed.dtype == torch.int32
    assert m.sign_packed.shape == (40, 3) and m.sign_packed.dtype == torch.int32
    assert m.mx.shape == (40,) and m.mx.dtype == torch.float32
    assert m.bias.shape == (40,) and m.bias.dtype == torch.float32
    assert m.alpha == float(np.float32(0.73))
    assert set(m.state_dict()) == {"packed", "sign_packed", "mx", "bias"}
    assert OPQLinear(64, 8, bias=False).bias is None
    assert "alpha=0.73" in repr(m)


@pytest.mark.parametrize("args", [(100, 8), (0, 8), (64, 0)])
def test_shape_checks(args):
    with pytest.raises(ValueError):
        OPQLinear(*args)


@pytest.mark.parametrize("alpha", [0.0, -1.0, float("nan"), float("inf")])
def test_alpha_checks(alpha):
    with pytest.raises(ValueError):
        OPQLinear(64, 8, alpha=alpha)


def test_no_cpu_forward():
    """The layer has no CPU path: a forward on host buffers fails loudly."""
    m = _filled(64, 8, True, 0.73, 0)
    with pytest.raises(ValueError):
        m(torch.zeros(2, 64, dtype=torch.bfloat16))


def test_replace_refuses_host_weights_and_changes_nothing():
    model = nn.Sequential(nn.Linear(64, 32), nn.ReLU(), nn.Linear(32, 16))
    with pytest.raises(ValueError, match="GPU"):
        replace_with_opq(model)
    assert isinstance(model[0], nn.Linear) and isinstance(model[2], nn.Linear)


def test_replace_checks_bits():
    for bits in (2, 7, 8):
        with pytest.raises(ValueError):
            replace_with_opq(nn.Sequential(nn.Linear(64, 8)), bits=bits)
    with pytest.raises(ValueError, match="4-bit"):
        replace_with_opq(nn.Sequential(nn.Linear(64, 8)), bits=5, group_size=64)
    # a b-bit layer's buffers follow the bit stream layout
    lay = OPQLinear(96, 8, bits=5)
    assert tuple(lay.packed.shape) == (8, 96 * 5 // 32) and lay.bits == 5
    with pytest.raises(ValueError):
        OPQLinear(96, 8, bits=6, group_size=32)


def test_replace_skips_ineligible_layers_before_touching_weights():
    """Layers with in_features % 32 != 0 and names under `skip` are not
    targets, so a model made only of them needs no GPU and is left as is."""
    model = nn.Sequential(nn.Linear(48, 64), nn.Sequential(nn.Linear(64, 8)))
    assert replace_with_opq(model, skip=["1"]) == []
    assert isinstance(model[0], nn.Linear) and isinstance(model[1][0], nn.Linear)


def _skeleton():
    return nn.Sequential(nn.Linear(64, 96), nn.GELU(),
                         nn.Sequential(nn.Linear(96, 32, bias=False)), nn.Linear(32, 8))


def test_save_load_round_trip(tmp_path):
    src = _skeleton()
    src[0] = _filled(64, 96, True, 0.73, 1)
    src[2][0] = _filled(96, 32, False, 0.45, 2)   # another alpha, no bias
    path = str(tmp_path / "w.safetensors")
    assert save_opq(src, path) == ["0", "2.0"]

    dst = _skeleton()
    assert load_opq(dst, path) == ["0", "2.0"]
    assert isinstance(dst[0], OPQLinear) and isinstance(dst[2][0], OPQLinear)
    assert isinstance(dst[3], nn.Linear)          # not in the file: untouched
    for a, b in ((src[0], dst[0]), (src[2][0], dst[2][0])):
        assert a.alpha == b.alpha
        sa, sb = a.state_dict(), b.state_dict()
        assert set(sa) == set(sb)
        for key in sa:
            assert torch.equal(sa[key], sb[key]), key
    assert dst[2][0].bias is None

    # loading again over OPQLinear layers replaces them the same way
    assert load_opq(dst, path) == ["0", "2.0"]
    assert torch.equal(dst[0].packed, src[0].packed)


def test_file_is_plain_tensors_with_a_json_header(tmp_path):
    from safetensors import safe_open
    src = nn.Sequential(_filled(64, 16, True, 1.0, 3))
    path = str(tmp_path / "w.safetensors")
    save_opq(src, path)
    with safe_open(path, framework="pt") as f:
        meta = json.loads(f.metadata()["opq"])
        assert meta["format"] == FORMAT
        assert meta["layers"]["0"] == {"in": 64, "out": 16, "alpha": 1.0, "bias": True, "group": 0,
                                       "bits": 4}
        assert sorted(f.keys()) == ["0.bias", "0.mx", "0.packed", "0.sign_packed"]


def test_load_checks_shapes_and_format(tmp_path):
    src = nn.Sequential(_filled(64, 16, True, 0.73, 4))
    path = str(tmp_path / "w.safetensors")
    save_opq(src, path)
    with pytest.raises(ValueError, match="16x64"):
        load_opq(nn.Sequential(nn.Linear(64, 24)), path)
    with pytest.raises(ValueError, match="not a Linear"):
        load_opq(nn.Sequential(nn.ReLU()), path)
    from safetensors.torch import save_file
    other = str(tmp_path / "other.safetensors")
    save_file({"x": torch.zeros(2)}, other)
    with pytest.raises(ValueError, match="format"):
        load_opq(nn.Sequential(nn.Linear(64, 16)), other)


def test_grouped_layer_buffers_and_round_trip(tmp_path):
    m = OPQLinear(256, 24, bias=False, alpha=0.73, group_size=64)
    assert m.mx.shape == (24, 4) and m.mx.dtype == torch.float16
    assert "group_size=64" in repr(m)
    g = torch.Generator().manual_seed(5)
    m.packed.copy_(torch.randint(-2**31, 2**31 - 1, m.packed.shape, dtype=torch.int32, generator=g))
    m.mx.copy_(torch.rand(m.mx.shape, generator=g).half())
    path = str(tmp_path / "g.safetensors")
    save_opq(nn.Sequential(m), path)
    dst = nn.Sequential(nn.Linear(256, 24, bias=False))
    load_opq(dst, path)
    assert dst[0].group_size == 64 and dst[0].mx.dtype == torch.float16
    assert torch.equal(dst[0].mx, m.mx) and torch.equal(dst[0].packed, m.packed)


@pytest.mark.parametrize("gs", [16, 48, 512])
def test_group_size_checks(gs):
    with pytest.raises(ValueError):
        OPQLinear(512, 8, group_size=gs)
    with pytest.raises(ValueError):
        replace_with_opq(nn.Sequential(nn.Linear(512, 8)), group_size=gs)


def test_grouped_replace_skips_layers_the_group_does_not_tile():
    model = nn.Sequential(nn.Linear(96, 8))      # 96 is no multiple of 64
    assert replace_with_opq(model, group_size=64) == []
