"""Seeded synthetic workloads shaped like a ~6B-parameter diffusion transformer.

These generators only draw numbers: they hold none of the quantizer's
arithmetic, and both the tests' oracle side and the GPU side get their inputs
from here.  Every host tensor is drawn with numpy's PCG64 ``default_rng(seed)``
in float64, cast to float32, and (for bf16 tensors) rounded to bfloat16 by
torch's cast; ``student_t_device`` draws the whole-model weights on the GPU.  Hidden size 3840, fused QKV 11520, FFN 10240 (up and gate fused to
20480), 30 blocks: the model card's Z-Image transformer is a 6.02B-parameter DiT
but the card gives no layer shapes, so these shapes stand in for it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Tuple

import numpy as np
import torch

ALPHA = 0.73           # the card's alpha for Z-Image
ALPHAS_SWEEP = (0.45, 0.73, 1.0)
HIDDEN = 3840
QKV = 3 * HIDDEN       # 11520
FFN = 10240
FFN_UPGATE = 2 * FFN   # 20480
BLOCKS = 30


# ------------------------------------------------------------------ distributions

def student_t(seed: int, shape, std: float = 0.02, nu: float = 4.0) -> np.ndarray:
    """Student-t(nu) scaled to standard deviation std (Var t_nu = nu/(nu-2))."""
    rng = np.random.default_rng(seed)
    s = std / math.sqrt(nu / (nu - 2.0))
    return (rng.standard_t(nu, size=shape) * s).astype(np.float32)


def student_t_outliers(seed: int, shape, std: float = 0.02, p: float = 0.001,
                       gain: float = 20.0) -> np.ndarray:
    """Student-t(4) at std, then a Bernoulli(p) mask multiplies entries by gain."""
    rng = np.random.default_rng(seed)
    s = std / math.sqrt(2.0)
    w = rng.standard_t(4.0, size=shape) * s
    mask = rng.random(shape) < p
    w[mask] *= gain
    return w.astype(np.float32)


def normal_laplace(seed: int, shape, std: float = 0.02, p_tail: float = 0.01,
                   b: float = 0.02) -> np.ndarray:
    """N(0, std^2) with probability 1 - p_tail, Laplace(0, b) otherwise."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(shape) * std
    tail = rng.random(shape) < p_tail
    w[tail] = rng.laplace(0.0, b, size=int(tail.sum()))
    return w.astype(np.float32)


def student_t_device(seed: int, shape, device, std: float = 0.02, nu: int = 4) -> torch.Tensor:
    """Student-t(nu) at standard deviation std drawn on `device` as bfloat16:
    z / sqrt(chi2_nu / nu), with z and the nu squared normals of chi2 from
    torch's generator seeded with `seed` (Philox on the GPU).  The same
    distribution as ``student_t`` but other numbers; it serves the whole-model
    workload, whose 5.3 B values would take minutes to draw on the host."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn(shape, device=device, generator=g)
    chi2 = torch.zeros(shape, device=device)
    for _ in range(nu):
        chi2.add_(torch.randn(shape, device=device, generator=g).square_())
    w = z.mul_(torch.rsqrt(chi2.div_(nu))).mul_(std / math.sqrt(nu / (nu - 2.0)))
    del chi2
    return w.to(torch.bfloat16)


def normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * std).astype(np.float32)


# ------------------------------------------------------------------ bf16 helpers

def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 ndarray -> CPU bfloat16 tensor (torch's round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> uint16 bit patterns (numpy, host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u32(t: torch.Tensor) -> np.ndarray:
    """int32 tensor holding uint32 words -> numpy uint32 (host)."""
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


# ------------------------------------------------------------------ configs

@dataclass
class Layer:
    name: str
    n: int
    k: int
    make_w: Callable[[], np.ndarray]     # float32 values before the bf16 cast
    w_dtype: str = "bf16"                 # "bf16" or "f32"
    m: int = 0                            # tokens of the paired activation (0: none)
    make_x: Callable[[], np.ndarray] = None

    @property
    def weights(self) -> int:
        return self.n * self.k


@dataclass
class Config:
    key: str
    title: str
    layers: List[Layer]
    alphas: Tuple[float, ...] = (ALPHA,)
    notes: Dict[str, str] = field(default_factory=dict)


def _c1() -> Config:
    return Config("tiny", "tiny oracle check: fp32 W 256x256 ~ N(0, 0.02^2), x bf16 [8, 256]", [
        Layer("w", 256, 256, lambda: normal(0, (256, 256), 0.02), "f32", 8,
              lambda: normal(1, (8, 256))),
    ])


def _c2() -> Config:
    return Config("skinny", "skinny linear: W 3840x3840 Student-t(4) std 0.02, x bf16 [32, 3840]", [
        Layer("w", HIDDEN, HIDDEN, lambda: student_t(2000, (HIDDEN, HIDDEN)), "bf16", 32,
              lambda: normal(2001, (32, HIDDEN))),
    ])


def _c3() -> Config:
    return Config("qkv", "DiT QKV projection: x bf16 [4096, 3840], W 11520x3840 Student-t(4) "
                  "std 0.02 with 0.1% x20 outliers", [
        Layer("qkv", QKV, HIDDEN, lambda: student_t_outliers(3000, (QKV, HIDDEN)), "bf16", 4096,
              lambda: normal(3001, (4096, HIDDEN))),
    ])


def _c4() -> Config:
    return Config("ffn", "DiT FFN pair: up/gate x[4096,3840] W 20480x3840; down x[4096,10240] "
                  "W 3840x10240; N(0, 0.02^2) with 1% Laplace(0, 0.02) tails", [
        Layer("up_gate", FFN_UPGATE, HIDDEN, lambda: normal_laplace(4000, (FFN_UPGATE, HIDDEN)),
              "bf16", 4096, lambda: normal(4002, (4096, HIDDEN))),
        Layer("down", HIDDEN, FFN, lambda: normal_laplace(4001, (HIDDEN, FFN)), "bf16", 4096,
              lambda: normal(4003, (4096, FFN))),
    ])


BLOCK_LAYERS = (("qkv", QKV, HIDDEN), ("o", HIDDEN, HIDDEN), ("up_gate", FFN_UPGATE, HIDDEN),
                ("down", HIDDEN, FFN))


def model_seed(block: int, layer: int) -> int:
    """Seed of layer `layer` (0..3: QKV, O, up/gate, down) of block `block`."""
    return 5000 + 4 * block + layer


def _c5(blocks: int = BLOCKS) -> Config:
    layers = []
    for b in range(blocks):
        for i, (nm, n, k) in enumerate(BLOCK_LAYERS):
            seed = model_seed(b, i)
            layers.append(Layer(f"block{b}.{nm}", n, k,
                                (lambda s=seed, n=n, k=k: student_t(s, (n, k))), "bf16"))
    return Config("model", f"whole-model quantize/dequant pass: {blocks} DiT blocks "
                  "(QKV 11520x3840, O 3840x3840, FFN 20480x3840 + 3840x10240), "
                  "Student-t(4) std 0.02", layers, alphas=ALPHAS_SWEEP)


CONFIGS = {"tiny": _c1, "skinny": _c2, "qkv": _c3, "ffn": _c4, "model": _c5}


def config(key: str, **kw) -> Config:
    return CONFIGS[key](**kw)


def model_weights(blocks: int = BLOCKS) -> int:
    return blocks * sum(n * k for _, n, k in BLOCK_LAYERS)
