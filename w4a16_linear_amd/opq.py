"""Python binding of libopq (include/opq.h): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels; this module
checks tensor placement, allocates outputs with torch on the caller's device
and passes raw pointers plus the current torch stream.  It never computes the
method itself and fails loudly when libopq.so is missing.

Packed words and sign words are carried in torch.int32 tensors holding the
uint32 bit patterns; bfloat16 tensors are passed by their bits.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libopq.so")
ABI_VERSION = 6

OPQ_F32 = 0
OPQ_BF16 = 1

# int opq_*(...) signatures, in header order
_SIGNATURES = {
    "opq_abi_version": (ctypes.c_int, []),
    "opq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "opq_decision_points": (ctypes.c_int, [ctypes.c_float, ctypes.c_void_p]),
    "opq_levels": (ctypes.c_int, [ctypes.c_float, ctypes.c_void_p]),
    "opq_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]),
    "opq_error_sums": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),
    "opq_dequantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "opq_linear_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                     ctypes.c_int64]),
    "opq_linear": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]),
    "opq_quantize_bits": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]),
    "opq_dequantize_bits": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),
    "opq_error_sums_bits": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_void_p]),
    "opq_linear_bits_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                          ctypes.c_int64, ctypes.c_int]),
    "opq_linear_bits": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "opq_linear_bits_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_void_p]),
    "opq_quantize_grouped": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]),
    "opq_dequantize_grouped": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),
    "opq_linear_grouped": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
}

_lib: Optional[ctypes.CDLL] = None


class OpqError(ValueError):
    """A libopq call returned a non-zero status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: status {status}: {text}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libopq.so once; raise if it is missing or of another ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libopq.so not built at {path}: run `python -m w4a16_linear_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    ver = lib.opq_abi_version()
    if ver != ABI_VERSION:
        raise RuntimeError(f"libopq ABI {ver}, binding expects {ABI_VERSION}")
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().opq_status_str(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise OpqError(fn, status, status_str(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need_cuda(name: str, t: torch.Tensor, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


# ------------------------------------------------------------------ host tables

def decision_points(alpha: float) -> np.ndarray:
    """The fifteen binary32 decision points the quantize kernel uses (host)."""
    out = np.zeros(15, np.float32)
    _check("opq_decision_points", load().opq_decision_points(alpha, out.ctypes.data))
    return out


def levels(alpha: float) -> np.ndarray:
    """The sixteen reconstruction levels (q/15)^(1/alpha) in double (host)."""
    out = np.zeros(16, np.float64)
    _check("opq_levels", load().opq_levels(alpha, out.ctypes.data))
    return out


# ------------------------------------------------------------------ device calls

class QuantizedWeight(NamedTuple):
    packed: torch.Tensor  # int32 [n, k/8]: eight 4-bit codes per word
    sign: torch.Tensor    # int32 [n, k/32]: sign plane
    scale: torch.Tensor   # float32 [n]: per-row max |w|

    @property
    def shape(self):
        return (self.packed.shape[0], self.packed.shape[1] * 8)


class BitsWeight(NamedTuple):
    """b-bit codes (3..6) with one float32 max per row; codes of a row form a
    little-endian bit stream along k (32 codes per `bits` words)."""
    packed: torch.Tensor  # int32 [n, k*bits/32]
    sign: torch.Tensor    # int32 [n, k/32]
    scale: torch.Tensor   # float32 [n]
    bits: int

    @property
    def shape(self):
        return (self.packed.shape[0], self.sign.shape[1] * 32)


class GroupedWeight(NamedTuple):
    """The group-wise stored form: one float16 max per `group` weights along k."""
    packed: torch.Tensor   # int32 [n, k/8]
    sign: torch.Tensor     # int32 [n, k/32]
    scale16: torch.Tensor  # float16 [n, k/group]: stored group maxima
    group: int             # 32, 64, 128 or 256

    @property
    def shape(self):
        return (self.packed.shape[0], self.packed.shape[1] * 8)


def quantize(w: torch.Tensor, alpha: float, out: Optional[QuantizedWeight] = None) -> QuantizedWeight:
    """Quantize a float32 or bfloat16 weight [n, k] on its device."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    _need_cuda("w", w, w.dtype, 2)
    n, k = w.shape
    if out is None:
        out = QuantizedWeight(
            torch.empty((n, k // 8), dtype=torch.int32, device=w.device),
            torch.empty((n, k // 32), dtype=torch.int32, device=w.device),
            torch.empty((n,), dtype=torch.float32, device=w.device))
    dtype = OPQ_BF16 if w.dtype == torch.bfloat16 else OPQ_F32
    st = load().opq_quantize(_ptr(w), dtype, n, k, alpha, _ptr(out.packed), _ptr(out.sign),
                             _ptr(out.scale), _stream(w.device))
    _check("opq_quantize", st)
    return out


def quantize_bits(w: torch.Tensor, alpha: float, bits: int,
                  out: Optional[BitsWeight] = None) -> BitsWeight:
    """Quantize a float32 or bfloat16 weight [n, k] with b-bit codes (3..6)."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    _need_cuda("w", w, w.dtype, 2)
    n, k = w.shape
    if bits not in (3, 4, 5, 6):
        raise ValueError(f"bits must be 3, 4, 5 or 6, got {bits}")
    if out is None:
        out = BitsWeight(torch.empty((n, k * bits // 32), dtype=torch.int32, device=w.device),
                         torch.empty((n, k // 32), dtype=torch.int32, device=w.device),
                         torch.empty((n,), dtype=torch.float32, device=w.device), bits)
    _check_bits(out, n, k)
    dtype = OPQ_BF16 if w.dtype == torch.bfloat16 else OPQ_F32
    st = load().opq_quantize_bits(_ptr(w), dtype, n, k, out.bits, alpha, _ptr(out.packed),
                                  _ptr(out.sign), _ptr(out.scale), _stream(w.device))
    _check("opq_quantize_bits", st)
    return out


def _check_bits(bw: BitsWeight, n: int, k: int) -> None:
    for name, t, dt in (("packed", bw.packed, torch.int32), ("sign", bw.sign, torch.int32)):
        _need_cuda(name, t, dt, 2)
    _need_cuda("scale", bw.scale, torch.float32, 1)
    if (bw.bits not in (3, 4, 5, 6) or tuple(bw.packed.shape) != (n, k * bw.bits // 32) or
            tuple(bw.sign.shape) != (n, k // 32) or tuple(bw.scale.shape) != (n,)):
        raise ValueError(f"b-bit weight buffers do not match n={n}, k={k}, bits={bw.bits}")


def quantize_grouped(w: torch.Tensor, alpha: float, group: int = 128,
                     out: Optional[GroupedWeight] = None) -> GroupedWeight:
    """Quantize a float32 or bfloat16 weight [n, k] to the group-wise form."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    _need_cuda("w", w, w.dtype, 2)
    n, k = w.shape
    if group not in (32, 64, 128, 256) or k % group:
        raise ValueError(f"group must be 32, 64, 128 or 256 and divide k={k}, got {group}")
    if out is None:
        out = GroupedWeight(
            torch.empty((n, k // 8), dtype=torch.int32, device=w.device),
            torch.empty((n, k // 32), dtype=torch.int32, device=w.device),
            torch.empty((n, k // group), dtype=torch.float16, device=w.device), group)
    _check_grouped(out, n, k)
    dtype = OPQ_BF16 if w.dtype == torch.bfloat16 else OPQ_F32
    st = load().opq_quantize_grouped(_ptr(w), dtype, n, k, out.group, alpha, _ptr(out.packed),
                                     _ptr(out.sign), _ptr(out.scale16), _stream(w.device))
    _check("opq_quantize_grouped", st)
    return out


def _check_grouped(gw: GroupedWeight, n: int, k: int) -> None:
    for name, t, dt in (("packed", gw.packed, torch.int32), ("sign", gw.sign, torch.int32),
                        ("scale16", gw.scale16, torch.float16)):
        _need_cuda(name, t, dt, 2)
    if (tuple(gw.packed.shape) != (n, k // 8) or tuple(gw.sign.shape) != (n, k // 32) or
            gw.group not in (32, 64, 128, 256) or tuple(gw.scale16.shape) != (n, k // gw.group)):
        raise ValueError(f"grouped weight buffers do not match n={n}, k={k}, group={gw.group}")


def dequantize(qw, alpha: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bfloat16 reconstruction [n, k] of a QuantizedWeight, GroupedWeight or
    BitsWeight."""
    n, k = qw.shape
    if isinstance(qw, BitsWeight):
        _check_bits(qw, n, k)
        if out is None:
            out = torch.empty((n, k), dtype=torch.bfloat16, device=qw.packed.device)
        _need_cuda("out", out, torch.bfloat16, 2)
        st = load().opq_dequantize_bits(_ptr(qw.packed), _ptr(qw.sign), _ptr(qw.scale), n, k,
                                        qw.bits, alpha, _ptr(out), _stream(qw.packed.device))
        _check("opq_dequantize_bits", st)
        return out
    if isinstance(qw, BitsWeight):
        _check_bits(qw, n, k)
        st = load().opq_linear_bits(_ptr(x), _ptr(qw.packed), _ptr(qw.sign), _ptr(qw.scale),
                                    _ptr(bias), m, n, k, qw.bits, alpha, _ptr(out), y_dtype,
                                    _ptr(workspace), ws_bytes, _stream(x.device))
        _check("opq_linear_bits", st)
        return out
    if isinstance(qw, GroupedWeight):
        _check_grouped(qw, n, k)
        if out is None:
            out = torch.empty((n, k), dtype=torch.bfloat16, device=qw.packed.device)
        _need_cuda("out", out, torch.bfloat16, 2)
        st = load().opq_dequantize_grouped(_ptr(qw.packed), _ptr(qw.sign), _ptr(qw.scale16), n, k,
                                           qw.group, alpha, _ptr(out), _stream(qw.packed.device))
        _check("opq_dequantize_grouped", st)
        return out
    for name, t, dt in (("packed", qw.packed, torch.int32), ("sign", qw.sign, torch.int32)):
        _need_cuda(name, t, dt, 2)
    _need_cuda("scale", qw.scale, torch.float32, 1)
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=qw.packed.device)
    st = load().opq_dequantize(_ptr(qw.packed), _ptr(qw.sign), _ptr(qw.scale), n, k, alpha,
                               _ptr(out), _stream(qw.packed.device))
    _check("opq_dequantize", st)
    return out


def linear_workspace_bytes(m: int, n: int, k: int, bits: int = 4) -> int:
    """Workspace bytes of opq_linear (bits = 4) or opq_linear_bits."""
    if bits == 4:
        return int(load().opq_linear_workspace_bytes(m, n, k))
    return int(load().opq_linear_bits_workspace_bytes(m, n, k, bits))


def error_sums(w: torch.Tensor, alpha: float, out: Optional[torch.Tensor] = None,
               bits: int = 4) -> torch.Tensor:
    """Per row of w: (sum w^2, sum (w - w')^2) as float64 [n, 2], w' the bf16
    reconstruction quantize + dequantize would give with b-bit codes (nothing
    stored)."""
    _need_cuda("w", w, w.dtype, 2)
    if w.dtype == torch.float32:
        dt = OPQ_F32
    elif w.dtype == torch.bfloat16:
        dt = OPQ_BF16
    else:
        raise ValueError(f"w must be float32 or bfloat16, got {w.dtype}")
    n, k = w.shape
    if out is None:
        out = torch.empty((n, 2), dtype=torch.float64, device=w.device)
    _need_cuda("out", out, torch.float64, 2)
    st = load().opq_error_sums_bits(_ptr(w), dt, n, k, bits, alpha, _ptr(out), _stream(w.device))
    _check("opq_error_sums_bits", st)
    return out


def snr_db(weights, alpha: float, bits: int = 4) -> float:
    """10 log10(sum w^2 / sum (w - w')^2) over one tensor or a list of tensors."""
    if isinstance(weights, torch.Tensor):
        weights = [weights]
    tot = None
    for w in weights:
        s = error_sums(w, alpha, bits=bits).sum(dim=0)
        tot = s if tot is None else tot + s
    num, den = (float(v) for v in tot.cpu())
    return float("inf") if den == 0.0 else 10.0 * float(np.log10(num / den))


# One workspace per device, grown on demand.  The linear calls overwrite what
# they use and need nothing in it initialised, so calls in one stream can share
# it; calls that may overlap (other streams) must pass workspaces of their own.
_workspaces: dict = {}


def shared_workspace(device: torch.device, nbytes: int) -> Optional[torch.Tensor]:
    """The per-device workspace, at least `nbytes` long (None for 0)."""
    if nbytes <= 0:
        return None
    key = torch.device(device).index if torch.device(device).index is not None \
        else torch.cuda.current_device()
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=torch.device("cuda", key))
        _workspaces[key] = ws
    return ws


def linear(x: torch.Tensor, qw, alpha: float, bias: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """y[m, n] = x[m, k] W'^T (+ bias), W' made from qw: a QuantizedWeight or a
    GroupedWeight (decoded on chip) or a BitsWeight (3, 5 or 6 bits: decoded
    into the workspace, then a dense bf16 product).

    out_dtype is torch.float32 or torch.bfloat16 (the float32 result rounded
    to nearest even).  `workspace`, when given, must be a uint8 device tensor
    of at least linear_workspace_bytes(m, n, k) bytes (its contents are
    overwritten); by default the per-device shared one is used.
    """
    _need_cuda("x", x, torch.bfloat16, 2)
    m, k = x.shape
    n, kw = qw.shape
    if kw != k:
        raise ValueError(f"x has k={k}, weight has k={kw}")
    if bias is not None:
        _need_cuda("bias", bias, torch.float32, 1)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    if out.dtype == torch.float32:
        y_dtype = OPQ_F32
    elif out.dtype == torch.bfloat16:
        y_dtype = OPQ_BF16
    else:
        raise ValueError(f"out must be float32 or bfloat16, got {out.dtype}")
    _need_cuda("out", out, out.dtype, 2)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must have shape {(m, n)}, got {tuple(out.shape)}")
    need = linear_workspace_bytes(m, n, k, qw.bits if isinstance(qw, BitsWeight) else 4)
    if workspace is None:
        workspace = shared_workspace(x.device, need)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA (HIP) tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if isinstance(qw, BitsWeight):
        _check_bits(qw, n, k)
        st = load().opq_linear_bits(_ptr(x), _ptr(qw.packed), _ptr(qw.sign), _ptr(qw.scale),
                                    _ptr(bias), m, n, k, qw.bits, alpha, _ptr(out), y_dtype,
                                    _ptr(workspace), ws_bytes, _stream(x.device))
        _check("opq_linear_bits", st)
        return out
    if isinstance(qw, GroupedWeight):
        _check_grouped(qw, n, k)
        st = load().opq_linear_grouped(_ptr(x), _ptr(qw.packed), _ptr(qw.sign), _ptr(qw.scale16),
                                       _ptr(bias), m, n, k, qw.group, alpha, _ptr(out), y_dtype,
                                       _ptr(workspace), ws_bytes, _stream(x.device))
        _check("opq_linear_grouped", st)
        return out
    st = load().opq_linear(_ptr(x), _ptr(qw.packed), _ptr(qw.sign), _ptr(qw.scale), _ptr(bias),
                           m, n, k, alpha, _ptr(out), y_dtype, _ptr(workspace), ws_bytes,
                           _stream(x.device))
    _check("opq_linear", st)
    return out


def linear_noalloc(x: torch.Tensor, bw: "BitsWeight", alpha: float,
                   bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """opq_linear_bits_noalloc: the b-bit linear layer with the library's fixed
    per-GPU scratch instead of a workspace (no device allocation in the call
    when `out` is given)."""
    _need_cuda("x", x, torch.bfloat16, 2)
    m, k = x.shape
    n, kw = bw.shape
    if kw != k:
        raise ValueError(f"x has k={k}, weight has k={kw}")
    _check_bits(bw, n, k)
    if bias is not None:
        _need_cuda("bias", bias, torch.float32, 1)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out must be float32 or bfloat16, got {out.dtype}")
    _need_cuda("out", out, out.dtype, 2)
    if tuple(out.shape) != (m, n):
        raise ValueError(f"out must have shape {(m, n)}, got {tuple(out.shape)}")
    y_dtype = OPQ_F32 if out.dtype == torch.float32 else OPQ_BF16
    st = load().opq_linear_bits_noalloc(_ptr(x), _ptr(bw.packed), _ptr(bw.sign), _ptr(bw.scale),
                                        _ptr(bias), m, n, k, bw.bits, alpha, _ptr(out), y_dtype,
                                        _stream(x.device))
    _check("opq_linear_bits_noalloc", st)
    return out
