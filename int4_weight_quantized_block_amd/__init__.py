"""MI355X (gfx950) ConvRot INT4 weight-quantized linear layer.

Thin Python binding over the C-ABI library ``libw4.so`` (declared in
``include/w4.h``).  The functions carry the C names and only marshal arguments:
they check dtypes / devices / contiguity, allocate the output tensors with torch,
and pass raw device pointers plus torch's current HIP stream.  Every step of the
layer runs in the library's HIP kernels; there is no Python or CPU fallback, and
importing a missing or unloadable library raises immediately on first use.

The layer (ComfyUI-INT-Crush README, "Inference / INT4" and "Forward Pass";
stable-diffusion.cpp PR #2010, "Summary"): block-Hadamard rotation of the
activations along K in groups of g (64 or 256), per-token int8 / int4
quantization, packed int4 weights with per-row scales (and zero points),
int32 GEMM, fused dequant (+ optional low-rank branch, + bias) to bf16.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "W4Error", "library_path", "load_library", "w4_pack_weights", "w4_rotate_quant_act",
    "w4_linear_cached_rot", "w4_linear", "w4_lowrank_down", "w4_workspace_bytes",
    "w4_linear_workspace_bytes", "w4_linear_fused", "LowRank", "RotationCache", "W4_OK", "W4_ERR_INVALID_ARG",
    "W4_ERR_SHAPE", "W4_ERR_UNSUPPORTED", "W4_ERR_ALIGN", "W4_ERR_HIP", "W4_ERR_WORKSPACE",
    "W4_MAX_K", "EXPORTS", "w4_probe_mfma_rate",
]

W4_OK, W4_ERR_INVALID_ARG, W4_ERR_SHAPE, W4_ERR_UNSUPPORTED, W4_ERR_ALIGN, W4_ERR_HIP, \
    W4_ERR_WORKSPACE = range(7)
W4_F32, W4_BF16 = 0, 1
W4_SYM, W4_ASYM = 0, 1
W4_OUT_BF16, W4_OUT_I32 = 0, 1
W4_MAX_K = 32768

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libw4.so")


class W4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _LowRankC(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("l1", ctypes.c_void_p), ("t", ctypes.c_void_p),
                ("l2", ctypes.c_void_p), ("r", ctypes.c_int)]


_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/w4.h
EXPORTS = {
    "w4_pack_weights": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P]),
    "w4_rotate_quant_act": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P]),
    "w4_linear_cached_rot": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _I, ctypes.POINTER(_LowRankC),
                                  _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "w4_linear": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P, _I, ctypes.POINTER(_LowRankC),
                       _I64, _P, _I, _P, _SZ, _P]),
    "w4_lowrank_down": (_I, [_P, _P, _I64, _I64, _I, _P, _P]),
    "w4_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _I]),
    "w4_linear_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _I]),
    "w4_linear_fused": (_I, [_I64, _I64, _I64, _I, _I, _I]),
    "w4_status_string": (ctypes.c_char_p, [_I]),
    "w4_last_error": (ctypes.c_char_p, []),
    "w4_version": (ctypes.c_char_p, []),
    "w4_probe_mfma_rate": (_I, [_I64, _I, _I, _P, _P]),
}

_lib = None


def load_library():
    """Load libw4.so (built in-tree by ``__graft_entry__.build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError("libw4.so is not built (%s); run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != W4_OK:
        lib = load_library()
        raise W4Error(status, "%s: %s" % (lib.w4_status_string(status).decode(),
                                          lib.w4_last_error().decode()))


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _opt(t, name, dtypes):
    return None if t is None else _dev(t, name, dtypes)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _fdtype(t: torch.Tensor) -> int:
    return W4_BF16 if t.dtype == torch.bfloat16 else W4_F32


def w4_workspace_bytes(M, N, K, act_bits, r=0) -> int:
    return int(load_library().w4_workspace_bytes(M, N, K, act_bits, r))


def w4_linear_workspace_bytes(M, N, K, act_bits, r=0) -> int:
    return int(load_library().w4_linear_workspace_bytes(M, N, K, act_bits, r))


def w4_linear_fused(M, N, K, g, act_bits, x_dtype=torch.bfloat16) -> bool:
    """True when w4_linear on this shape runs as one fused rotate + quantize + GEMM kernel."""
    return bool(load_library().w4_linear_fused(M, N, K, g, act_bits, W4_BF16 if x_dtype == torch.bfloat16 else W4_F32))


def w4_pack_weights(W: torch.Tensor, g: int, asym: bool = False):
    """Rotate, quantize per row and pack W [N, K] (fp32 / bf16).

    Returns (packed uint8 [N, K/2], row_scale f32 [N], zp uint8 [N] or None)."""
    lib = load_library()
    _dev(W, "W", (torch.float32, torch.bfloat16))
    N, K = W.shape
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scale = torch.empty((N,), dtype=torch.float32, device=W.device)
    zp = torch.empty((N,), dtype=torch.uint8, device=W.device) if asym else None
    _check(lib.w4_pack_weights(W.data_ptr(), _fdtype(W), N, K, g, W4_ASYM if asym else W4_SYM,
                               packed.data_ptr(), scale.data_ptr(),
                               zp.data_ptr() if zp is not None else None, _stream(W.device)))
    return packed, scale, zp


def w4_rotate_quant_act(X: torch.Tensor, g: int, act_bits: int):
    """Rotate and quantize the tokens of X [M, K] (fp32 / bf16).

    Returns (q int8 [M, K] or packed uint8 [M, K/2], tok_scale f32 [M], tok_rowsum int32 [M])."""
    lib = load_library()
    _dev(X, "X", (torch.float32, torch.bfloat16))
    M, K = X.shape
    if act_bits == 8:
        q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    else:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    s = torch.empty((M,), dtype=torch.float32, device=X.device)
    rs = torch.empty((M,), dtype=torch.int32, device=X.device)
    _check(lib.w4_rotate_quant_act(X.data_ptr(), _fdtype(X), M, K, g, act_bits, q.data_ptr(),
                                   s.data_ptr(), rs.data_ptr(), _stream(X.device)))
    return q, s, rs


@dataclass
class LowRank:
    """Low-rank side branch (x . L1) . L2 on the unrotated input, added before the bias.

    Both factors are rank-major: ``l1`` = L1 transposed, bf16 [r, K]; ``l2`` = L2, bf16 [r, N].
    Give either ``t`` (f32 [M, r] = x . L1, e.g. from ``w4_lowrank_down``) or ``x`` and ``l1``."""
    l2: torch.Tensor
    x: Optional[torch.Tensor] = None
    l1: Optional[torch.Tensor] = None
    t: Optional[torch.Tensor] = None

    @property
    def r(self) -> int:
        return int(self.l2.shape[0])

    def as_c(self):
        c = _LowRankC()
        c.x = _opt(self.x, "lowrank.x", (torch.bfloat16,))
        c.l1 = _opt(self.l1, "lowrank.l1", (torch.bfloat16,))
        c.t = _opt(self.t, "lowrank.t", (torch.float32,))
        c.l2 = _dev(self.l2, "lowrank.l2", (torch.bfloat16,))
        c.r = self.r
        return c


def _y(M, N, out_i32, device, out):
    if out is not None:
        _dev(out, "out", (torch.int32,) if out_i32 else (torch.bfloat16,))
        if tuple(out.shape) != (M, N):
            raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (M, N)))
        return out
    return torch.empty((M, N), dtype=torch.int32 if out_i32 else torch.bfloat16, device=device)


def _ws(nbytes, device, ws):
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    return ws


def w4_linear_cached_rot(q, tok_scale, tok_rowsum, act_bits: int, packed, row_scale, zp=None,
                         bias=None, lowrank: Optional[LowRank] = None, out_i32: bool = False,
                         out=None, ws=None):
    """GEMM + fused dequant on codes from ``w4_rotate_quant_act``.  Returns Y [M, N]."""
    lib = load_library()
    _dev(q, "q", (torch.int8,) if act_bits == 8 else (torch.uint8,))
    _dev(tok_scale, "tok_scale", (torch.float32,))
    _dev(tok_rowsum, "tok_rowsum", (torch.int32,))
    _dev(packed, "packed", (torch.uint8,))
    _dev(row_scale, "row_scale", (torch.float32,))
    _opt(zp, "zp", (torch.uint8,))
    _opt(bias, "bias", (torch.float32, torch.bfloat16))
    M = tok_scale.shape[0]
    N, K = packed.shape[0], packed.shape[1] * 2
    Y = _y(M, N, out_i32, packed.device, out)
    lrc = lowrank.as_c() if lowrank is not None else None
    r = lowrank.r if (lowrank is not None and lowrank.t is None and not out_i32) else 0
    ws = _ws(w4_workspace_bytes(M, N, K, act_bits, r), packed.device, ws)
    _check(lib.w4_linear_cached_rot(
        q.data_ptr(), tok_scale.data_ptr(), tok_rowsum.data_ptr(), act_bits, packed.data_ptr(),
        row_scale.data_ptr(), zp.data_ptr() if zp is not None else None,
        bias.data_ptr() if bias is not None else None,
        _fdtype(bias) if bias is not None else W4_BF16,
        ctypes.byref(lrc) if lrc is not None else None, M, N, K, Y.data_ptr(),
        W4_OUT_I32 if out_i32 else W4_OUT_BF16,
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream(packed.device)))
    return Y


def w4_linear(X, g: int, act_bits: int, packed, row_scale, zp=None, bias=None,
              lowrank: Optional[LowRank] = None, out_i32: bool = False, out=None, ws=None):
    """The whole layer on X [M, K]: rotate + quantize, GEMM, fused dequant.  Returns Y [M, N]."""
    lib = load_library()
    _dev(X, "X", (torch.float32, torch.bfloat16))
    _dev(packed, "packed", (torch.uint8,))
    _dev(row_scale, "row_scale", (torch.float32,))
    _opt(zp, "zp", (torch.uint8,))
    _opt(bias, "bias", (torch.float32, torch.bfloat16))
    M, K = X.shape
    N = packed.shape[0]
    if packed.shape[1] * 2 != K:
        raise ValueError("packed is [%d, %d] but X has K=%d" % (N, packed.shape[1], K))
    Y = _y(M, N, out_i32, X.device, out)
    lrc = lowrank.as_c() if lowrank is not None else None
    r = lowrank.r if (lowrank is not None and lowrank.t is None and not out_i32) else 0
    ws = _ws(w4_linear_workspace_bytes(M, N, K, act_bits, r), X.device, ws)
    _check(lib.w4_linear(
        X.data_ptr(), _fdtype(X), M, K, g, act_bits, packed.data_ptr(), row_scale.data_ptr(),
        zp.data_ptr() if zp is not None else None, bias.data_ptr() if bias is not None else None,
        _fdtype(bias) if bias is not None else W4_BF16,
        ctypes.byref(lrc) if lrc is not None else None, N, Y.data_ptr(),
        W4_OUT_I32 if out_i32 else W4_OUT_BF16,
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream(X.device)))
    return Y


def w4_lowrank_down(x: torch.Tensor, l1: torch.Tensor) -> torch.Tensor:
    """t = x . L1 (f32 [M, r]) for a low-rank branch, shareable by linears reading x.

    ``l1`` is L1 transposed, bf16 [r, K] (rank-major, like a LoRA down weight)."""
    lib = load_library()
    _dev(x, "x", (torch.bfloat16,))
    _dev(l1, "l1", (torch.bfloat16,))
    M, K = x.shape
    r = l1.shape[0]
    if l1.dim() != 2 or l1.shape[1] != K:
        raise ValueError("l1 has shape %s, expected [r, %d]" % (tuple(l1.shape), K))
    t = torch.empty((M, r), dtype=torch.float32, device=x.device)
    _check(lib.w4_lowrank_down(x.data_ptr(), l1.data_ptr(), M, K, r, t.data_ptr(), _stream(x.device)))
    return t


def w4_probe_mfma_rate(blocks: int, iters: int, random_operands: bool, device="cuda") -> torch.Tensor:
    """Launch the int8 MFMA rate probe (a measurement tool, not a step of the layer) on the
    current stream; returns the checksum tensor it writes.  Work: blocks * 4 * iters * 4 *
    2 * 32**3 int ops."""
    lib = load_library()
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=device)
    _check(lib.w4_probe_mfma_rate(blocks, iters, 1 if random_operands else 0, sink.data_ptr(), _stream(sink.device)))
    return sink


class RotationCache:
    """Rotated + quantized activations shared by linears that read the same input.

    stable-diffusion.cpp PR #2010, "Summary": the activation rotation / quantize is
    shared and cached per (input, group size).  The key is the tensor's identity
    (storage pointer, offset, shape, strides, dtype), torch's in-place version counter,
    g and act_bits; the entry keeps a reference to the input, so its storage cannot be
    freed and reused while cached.  Scope it to one block / forward and ``clear()`` it."""

    def __init__(self):
        self._d = {}
        self.hits = 0
        self.misses = 0

    @staticmethod
    def _key(X: torch.Tensor, g: int, act_bits: int):
        return (X.data_ptr(), X.storage_offset(), tuple(X.shape), tuple(X.stride()), X.dtype,
                X._version, g, act_bits)

    def get(self, X: torch.Tensor, g: int, act_bits: int):
        k = self._key(X, g, act_bits)
        hit = self._d.get(k)
        if hit is not None:
            self.hits += 1
            return hit[1]
        self.misses += 1
        val = w4_rotate_quant_act(X, g, act_bits)
        self._d[k] = (X, val)
        return val

    def clear(self):
        self._d.clear()

    def __len__(self):
        return len(self._d)
