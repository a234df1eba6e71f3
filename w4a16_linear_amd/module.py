"""torch front end over libopq: an OPQ linear layer, in-place model conversion,
and save / load of the stored form.

Model card "OPQ INT4 Z-Image": the file list ("文件结构") names an OPQ module
holding an ``OPQLinear`` layer and ``replace_with_opq``; "在你自己的代码中使用"
converts a loaded model in place with ``replace_with_opq(model, bits=4,
alpha=0.73)``; "从量化权重加载的流程说明" rebuilds the ``OPQLinear`` structure
over a model skeleton and then overwrites its ``packed`` / ``sign_packed`` /
``mx`` buffers from saved files.  The buffers here keep those names.  ``mx``
is either one float32 max per output row, or (``group_size`` set) the card's
own form: one float16 max per group of ``group_size`` weights along the input
dimension ("技术细节 / 存储格式").  ``bits`` (the configuration section's
``OPQ_BITS``: 3, 4, 5 or 6) sets the code width; other than 4, ``packed``
holds the codes of a row as a bit stream along the input dimension.

Every step runs in libopq's kernels: a layer whose buffers are not on the GPU
raises instead of computing anywhere else.  Saved files are safetensors (plain
tensors plus a JSON header; loading executes nothing from the file).
"""
from __future__ import annotations

import json
from typing import Dict, Iterable, List, Optional

import numpy as np
import torch
from torch import nn

from . import opq

FORMAT = "opq-int4/1"
_META_KEY = "opq"


def _f32(alpha: float) -> float:
    """alpha as the binary32 value every libopq call receives."""
    a = float(np.float32(alpha))
    if not np.isfinite(a) or a <= 0.0:
        raise ValueError(f"alpha must be finite and > 0, got {alpha}")
    return a


class OPQLinear(nn.Module):
    """y = x W'^T (+ bias) with W' held as OPQ codes: `bits`-bit magnitudes
    (``packed`` [out, in*bits/32] int32; for 4 bits eight nibbles per word), a
    sign plane (``sign_packed`` [out, in/32] int32) and the maxima ``mx``:
    float32 [out] (one per output row), or, for 4 bits, float16
    [out, in/group_size] with ``group_size`` in 32, 64, 128, 256.  The bias,
    when present, is float32.  x may be bfloat16 or float32 (it is rounded to
    bfloat16, the layer's activation type); y has x's dtype."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 alpha: float = 0.73, device=None, group_size: Optional[int] = None,
                 bits: int = 4):
        super().__init__()
        if in_features <= 0 or in_features % 32:
            raise ValueError(f"in_features must be a positive multiple of 32, got {in_features}")
        if out_features <= 0:
            raise ValueError(f"out_features must be positive, got {out_features}")
        if group_size is not None and (group_size not in (32, 64, 128, 256) or
                                       in_features % group_size):
            raise ValueError(f"group_size must be 32, 64, 128 or 256 and divide in_features="
                             f"{in_features}, got {group_size}")
        if bits not in (3, 4, 5, 6):
            raise ValueError(f"bits must be 3, 4, 5 or 6, got {bits}")
        if group_size is not None and bits != 4:
            raise ValueError("group-wise maxima are built for 4-bit codes only")
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.alpha = _f32(alpha)
        self.group_size = group_size
        self.bits = int(bits)
        kw = dict(dtype=torch.int32, device=device)
        self.register_buffer("packed", torch.zeros((out_features, in_features * bits // 32), **kw))
        self.register_buffer("sign_packed", torch.zeros((out_features, in_features // 32), **kw))
        if group_size:
            self.register_buffer("mx", torch.zeros((out_features, in_features // group_size),
                                                   dtype=torch.float16, device=device))
        else:
            self.register_buffer("mx", torch.zeros((out_features,), dtype=torch.float32,
                                                   device=device))
        if bias:
            self.register_buffer("bias", torch.zeros((out_features,), dtype=torch.float32,
                                                     device=device))
        else:
            self.register_buffer("bias", None)

    # -- conversion ---------------------------------------------------------

    @classmethod
    def from_linear(cls, lin: nn.Linear, alpha: float = 0.73,
                    group_size: Optional[int] = None, bits: int = 4) -> "OPQLinear":
        """Quantize an nn.Linear whose weight is on the GPU (float32 or bfloat16)."""
        w = lin.weight.detach()
        if not w.is_cuda:
            raise ValueError("OPQLinear.from_linear: the weight must be on the GPU "
                             "(libopq has no CPU path)")
        if w.dtype not in (torch.float32, torch.bfloat16):
            w = w.float()
        out = cls(lin.in_features, lin.out_features, bias=lin.bias is not None, alpha=alpha,
                  device=w.device, group_size=group_size, bits=bits)
        if bits != 4:
            opq.quantize_bits(w.contiguous(), out.alpha, bits, out=out.qweight())
        elif group_size:
            opq.quantize_grouped(w.contiguous(), out.alpha, group_size, out=out.qweight())
        else:
            opq.quantize(w.contiguous(), out.alpha, out=out.qweight())
        if lin.bias is not None:
            out.bias.copy_(lin.bias.detach().float())
        return out

    def qweight(self):
        if self.bits != 4:
            return opq.BitsWeight(self.packed, self.sign_packed, self.mx, self.bits)
        if self.group_size:
            return opq.GroupedWeight(self.packed, self.sign_packed, self.mx, self.group_size)
        return opq.QuantizedWeight(self.packed, self.sign_packed, self.mx)

    def dequantized_weight(self) -> torch.Tensor:
        """W' as bfloat16 [out, in] (what the layer multiplies by)."""
        return opq.dequantize(self.qweight(), self.alpha)

    # -- forward ------------------------------------------------------------

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dim {self.in_features}, got {tuple(x.shape)}")
        if x.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"x must be bfloat16 or float32, got {x.dtype}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        y = opq.linear(x2, self.qweight(), self.alpha, bias=self.bias, out_dtype=x.dtype)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, alpha={self.alpha:.8g}, "
                f"group_size={self.group_size}, bits={self.bits}")


# ---------------------------------------------------------------- conversion

def _targets(model: nn.Module, skip: Iterable[str], group_size: Optional[int] = None):
    skip = tuple(skip)
    for parent_name, parent in model.named_modules():
        # every slot, also a second one holding a module already seen
        # (named_children would skip it)
        for cname, child in list(parent._modules.items()):
            full = f"{parent_name}.{cname}" if parent_name else cname
            if not isinstance(child, nn.Linear):
                continue
            if any(full == s or full.startswith(s + ".") for s in skip):
                continue
            if child.in_features % (group_size or 32):
                continue  # packed words (and groups) must tile the input dimension
            yield full, parent, cname, child


def replace_with_opq(model: nn.Module, bits: int = 4, alpha: float = 0.73,
                     skip: Iterable[str] = (), group_size: Optional[int] = None) -> List[str]:
    """Swap every nn.Linear of `model` (in place) for an OPQLinear holding its
    quantized weight; returns the qualified names replaced.  `group_size`
    None keeps one float32 max per output row; 32, 64, 128 or 256 stores the
    card's float16 max per group.  Layers whose in_features is not a multiple
    of 32 (and of the group), and names under `skip`, stay as they are.  A
    Linear reached under several names is quantized once and shared.  `bits`
    3, 5 or 6 stores b-bit codes (per-row maxima only); their forward pass
    decodes into a workspace before a dense product.  All eligible weights
    must be on the GPU: nothing is replaced otherwise."""
    if bits not in (3, 4, 5, 6):
        raise ValueError(f"bits must be 3, 4, 5 or 6, got {bits}")
    if group_size is not None and bits != 4:
        raise ValueError("group-wise maxima are built for 4-bit codes only")
    if group_size is not None and group_size not in (32, 64, 128, 256):
        raise ValueError(f"group_size must be 32, 64, 128 or 256, got {group_size}")
    alpha = _f32(alpha)
    found = list(_targets(model, skip, group_size))
    for full, _, _, child in found:
        if not child.weight.is_cuda:
            raise ValueError(f"replace_with_opq: {full}.weight is not on the GPU "
                             "(libopq has no CPU path); move the model first")
    made: Dict[int, OPQLinear] = {}
    for _, parent, cname, child in found:
        if id(child) not in made:
            made[id(child)] = OPQLinear.from_linear(child, alpha, group_size, bits)
        setattr(parent, cname, made[id(child)])
    return [full for full, _, _, _ in found]


# ---------------------------------------------------------------- save / load

def _opq_layers(model: nn.Module):
    seen = set()
    for name, mod in model.named_modules():
        if isinstance(mod, OPQLinear) and id(mod) not in seen:
            seen.add(id(mod))
            yield name, mod


def save_opq(model: nn.Module, path: str) -> List[str]:
    """Write every OPQLinear's buffers to a safetensors file; returns the
    layer names saved.  The header records the format, and per layer its
    shape, alpha, code width, group size and whether it has a bias.  A layer reached under several
    names is saved once, under the first."""
    from safetensors.torch import save_file

    tensors: Dict[str, torch.Tensor] = {}
    layers = {}
    for name, mod in _opq_layers(model):
        layers[name] = {"in": mod.in_features, "out": mod.out_features, "alpha": mod.alpha,
                        "bias": mod.bias is not None, "group": mod.group_size or 0,
                        "bits": mod.bits}
        for b in ("packed", "sign_packed", "mx") + (("bias",) if mod.bias is not None else ()):
            tensors[f"{name}.{b}"] = getattr(mod, b).detach().to("cpu").contiguous()
    meta = {_META_KEY: json.dumps({"format": FORMAT, "layers": layers})}
    save_file(tensors, path, metadata=meta)
    return list(layers)


def load_opq(model: nn.Module, path: str, device=None) -> List[str]:
    """Fill `model` from a file written by save_opq: each saved layer name must
    name an nn.Linear (a skeleton: its weights are dropped) or an OPQLinear of
    the same shape, which becomes an OPQLinear holding the saved buffers.  The
    buffers go to `device`, by default that of the module they replace.
    Returns the layer names loaded."""
    from safetensors import safe_open

    with safe_open(path, framework="pt", device="cpu") as f:
        meta = json.loads((f.metadata() or {}).get(_META_KEY, "null") or "null")
        if not meta or meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not an OPQ file of format {FORMAT}")
        layers = meta["layers"]
        for name, info in layers.items():
            parent_name, _, cname = name.rpartition(".")
            parent = model.get_submodule(parent_name) if parent_name else model
            old = getattr(parent, cname, None)
            if isinstance(old, OPQLinear):
                ref_dev = old.packed.device
            elif isinstance(old, nn.Linear):
                ref_dev = old.weight.device
            else:
                raise ValueError(f"{path}: {name} is not a Linear in this model")
            if (old.in_features, old.out_features) != (info["in"], info["out"]):
                raise ValueError(f"{path}: {name} is {info['out']}x{info['in']} in the file, "
                                 f"{old.out_features}x{old.in_features} in the model")
            dev = torch.device(device) if device is not None else ref_dev
            new = OPQLinear(info["in"], info["out"], bias=info["bias"], alpha=info["alpha"],
                            device=dev, group_size=info.get("group") or None,
                            bits=info.get("bits", 4))
            for b in ("packed", "sign_packed", "mx") + (("bias",) if info["bias"] else ()):
                t = f.get_tensor(f"{name}.{b}")
                dst = getattr(new, b)
                if t.shape != dst.shape or t.dtype != dst.dtype:
                    raise ValueError(f"{path}: {name}.{b} is {t.dtype}{tuple(t.shape)}, "
                                     f"expected {dst.dtype}{tuple(dst.shape)}")
                dst.copy_(t)
            # every slot holding the replaced module (a shared layer is saved once)
            for _, mod in list(model.named_modules()):
                for slot, child in list(mod._modules.items()):
                    if child is old:
                        setattr(mod, slot, new)
    return list(layers)
