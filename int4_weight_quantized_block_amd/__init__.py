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
from torch.autograd.graph import increment_version

__all__ = [
    "W4Error", "library_path", "load_library", "w4_pack_weights", "w4_rotate_quant_act",
    "w4_linear_cached_rot", "w4_linear", "w4_lowrank_down", "w4_workspace_bytes",
    "w4_linear_workspace_bytes", "w4_linear_fused", "LowRank", "RotationCache", "W4_OK", "W4_ERR_INVALID_ARG",
    "W4_ERR_SHAPE", "W4_ERR_UNSUPPORTED", "W4_ERR_ALIGN", "W4_ERR_HIP", "W4_ERR_WORKSPACE",
    "W4_MAX_K", "EXPORTS", "w4_linear_noalloc", "w4_noalloc_scratch_bytes",
    "w4_pack_weights_grouped", "w4_linear_cached_rot_grouped", "w4_linear_grouped",
    "w4_grouped_workspace_bytes", "w4_linear_grouped_workspace_bytes", "w4_rotate_quant_act_lowrank",
    "w4_rotate_quant_act_lowrank_fused", "w4_linear_cached_rot_multi", "LinearOut", "MULTI_MAX",
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
                ("l2", ctypes.c_void_p), ("r", ctypes.c_int), ("ldt", ctypes.c_int)]


_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t


class _LinearOutC(ctypes.Structure):
    _fields_ = [("packed", _P), ("row_scale", _P), ("zp", _P), ("bias", _P), ("bias_dtype", _I),
                ("lr", ctypes.POINTER(_LowRankC)), ("N", _I64), ("Y", _P), ("y_kind", _I)]

# name -> (restype, argtypes), mirroring include/w4.h
EXPORTS = {
    "w4_pack_weights": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P]),
    "w4_rotate_quant_act": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P]),
    "w4_linear_cached_rot": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _I, ctypes.POINTER(_LowRankC),
                                  _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "w4_linear_cached_rot_multi": (_I, [_P, _P, _P, _I, _I64, _I64, _I, ctypes.POINTER(_LinearOutC), _P, _SZ,
                                        _P]),
    "w4_linear": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P, _I, ctypes.POINTER(_LowRankC),
                       _I64, _P, _I, _P, _SZ, _P]),
    "w4_linear_noalloc": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P, _I, ctypes.POINTER(_LowRankC),
                               _I64, _P, _I, _P]),
    "w4_noalloc_scratch_bytes": (_SZ, []),
    "w4_pack_weights_grouped": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P]),
    "w4_linear_cached_rot_grouped": (_I, [_P, _P, _I, _P, _P, _I, _P, _I, ctypes.POINTER(_LowRankC),
                                          _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "w4_linear_grouped": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _I, _P, _I, ctypes.POINTER(_LowRankC),
                               _I64, _P, _I, _P, _SZ, _P]),
    "w4_grouped_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _I, _I]),
    "w4_linear_grouped_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _I, _I]),
    "w4_lowrank_down": (_I, [_P, _P, _I64, _I64, _I, _P, _P]),
    "w4_rotate_quant_act_lowrank": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P, _I, _P, _I64, _P]),
    "w4_rotate_quant_act_lowrank_fused": (_I, [_I64, _I]),
    "w4_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _I]),
    "w4_linear_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _I]),
    "w4_linear_fused": (_I, [_I64, _I64, _I64, _I, _I, _I]),
    "w4_status_string": (ctypes.c_char_p, [_I]),
    "w4_last_error": (ctypes.c_char_p, []),
    "w4_version": (ctypes.c_char_p, []),
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


def _shape(t, name: str, shape) -> None:
    """Raise ValueError unless tensor ``t`` (if given) has exactly ``shape``.

    The C ABI takes bare pointers and cannot see sizes, so every tensor is checked against
    (M, N, K, r) here, before anything is launched: a short bias or a mis-shaped code
    buffer would otherwise be read past its end by the kernels."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _matrix(t, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dim() != 2:
        raise ValueError("%s must be 2-D, got shape %s" % (name, tuple(t.shape)))
    return int(t.shape[0]), int(t.shape[1])


def _check_weights(packed, row_scale, zp, bias, N: int, K: int):
    _shape(packed, "packed", (N, K // 2))
    _shape(row_scale, "row_scale", (N,))
    _shape(zp, "zp", (N,))
    _shape(bias, "bias", (N,))


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
    N, K = _matrix(W, "W")
    _dev(W, "W", (torch.float32, torch.bfloat16))
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
    M, K = _matrix(X, "X")
    _dev(X, "X", (torch.float32, torch.bfloat16))
    if act_bits == 8:
        q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    else:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    s = torch.empty((M,), dtype=torch.float32, device=X.device)
    rs = torch.empty((M,), dtype=torch.int32, device=X.device)
    _check(lib.w4_rotate_quant_act(X.data_ptr(), _fdtype(X), M, K, g, act_bits, q.data_ptr(),
                                   s.data_ptr(), rs.data_ptr(), _stream(X.device)))
    return q, s, rs


def w4_rotate_quant_act_lowrank(X: torch.Tensor, g: int, act_bits: int, l1: torch.Tensor, t=None):
    """w4_rotate_quant_act and t = X . L1 in one pass over bf16 X [M, K].

    ``l1`` is bf16 [r, K] (L1 transposed; stack the factors of every linear that reads X).
    Returns (q, tok_scale, tok_rowsum, t f32 [M, r]); ``t`` may be given (a [M, r] f32 GPU
    tensor with unit column stride)."""
    lib = load_library()
    M, K = _matrix(X, "X")
    r = _matrix(l1, "l1")[0]
    _shape(l1, "l1", (r, K))
    _dev(X, "X", (torch.bfloat16,))
    _dev(l1, "l1", (torch.bfloat16,))
    if act_bits == 8:
        q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    else:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    s = torch.empty((M,), dtype=torch.float32, device=X.device)
    rs = torch.empty((M,), dtype=torch.int32, device=X.device)
    if t is None:
        t = torch.empty((M, r), dtype=torch.float32, device=X.device)
    _shape(t, "t", (M, r))
    tp = _strided_t(t)
    _check(lib.w4_rotate_quant_act_lowrank(X.data_ptr(), W4_BF16, M, K, g, act_bits, q.data_ptr(), s.data_ptr(),
                                           rs.data_ptr(), l1.data_ptr(), r, tp, int(t.stride(0)), _stream(X.device)))
    increment_version(t)
    return q, s, rs, t


def w4_rotate_quant_act_lowrank_fused(K: int, g: int) -> bool:
    return bool(load_library().w4_rotate_quant_act_lowrank_fused(K, g))


@dataclass
class LowRank:
    """Low-rank side branch (x . L1) . L2 on the unrotated input, added before the bias.

    Both factors are rank-major: ``l1`` = L1 transposed, bf16 [r, K]; ``l2`` = L2, bf16 [r, N].
    Give either ``t`` (f32 [M, r] = x . L1, e.g. from ``w4_lowrank_down``) or ``x`` and ``l1``.
    ``t`` may be a column range of a wider f32 tensor (unit column stride, any row stride),
    e.g. a slice of the t that ``w4_rotate_quant_act_lowrank`` computes for stacked factors."""
    l2: torch.Tensor
    x: Optional[torch.Tensor] = None
    l1: Optional[torch.Tensor] = None
    t: Optional[torch.Tensor] = None

    @property
    def r(self) -> int:
        return int(self.l2.shape[0])

    def check(self, M: int, N: int, K: int, need_t: bool) -> None:
        """Shapes against the layer: l2 [r, N]; t [M, r], or x [M, K] and l1 [r, K]."""
        r, n2 = _matrix(self.l2, "lowrank.l2")
        if n2 != N:
            raise ValueError("lowrank.l2 has shape %s, expected [r, %d]" % (tuple(self.l2.shape), N))
        if self.t is not None:
            _shape(self.t, "lowrank.t", (M, r))
        elif need_t:
            if self.x is None or self.l1 is None:
                raise ValueError("lowrank needs t, or x and l1")
            _shape(self.x, "lowrank.x", (M, K))
            _shape(self.l1, "lowrank.l1", (r, K))

    def as_c(self):
        c = _LowRankC()
        c.x = _opt(self.x, "lowrank.x", (torch.bfloat16,))
        c.l1 = _opt(self.l1, "lowrank.l1", (torch.bfloat16,))
        c.t = _strided_t(self.t) if self.t is not None else None
        c.l2 = _dev(self.l2, "lowrank.l2", (torch.bfloat16,))
        c.r = self.r
        c.ldt = int(self.t.stride(0)) if self.t is not None else 0
        return c


def _strided_t(t: torch.Tensor) -> int:
    """Device pointer of a low-rank t: f32, on the GPU, unit column stride (any row stride)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("lowrank.t must be a GPU tensor")
    if t.dtype != torch.float32:
        raise TypeError("lowrank.t has dtype %s, expected torch.float32" % t.dtype)
    if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise ValueError("lowrank.t must be [M, r] with unit column stride")
    return t.data_ptr()


def _y(M, N, out_i32, device, out):
    if out is not None:
        _shape(out, "out", (M, N))
        _dev(out, "out", (torch.int32,) if out_i32 else (torch.bfloat16,))
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
    if act_bits not in (4, 8):
        raise ValueError("act_bits must be 4 or 8, got %r" % (act_bits,))
    N, Kh = _matrix(packed, "packed")
    K = 2 * Kh
    M = _matrix(q, "q")[0]
    _shape(q, "q", (M, K) if act_bits == 8 else (M, K // 2))
    _shape(tok_scale, "tok_scale", (M,))
    _shape(tok_rowsum, "tok_rowsum", (M,))
    _check_weights(packed, row_scale, zp, bias, N, K)
    if lowrank is not None:
        lowrank.check(M, N, K, need_t=not out_i32)
    _dev(q, "q", (torch.int8,) if act_bits == 8 else (torch.uint8,))
    _dev(tok_scale, "tok_scale", (torch.float32,))
    _dev(tok_rowsum, "tok_rowsum", (torch.int32,))
    _dev(packed, "packed", (torch.uint8,))
    _dev(row_scale, "row_scale", (torch.float32,))
    _opt(zp, "zp", (torch.uint8,))
    _opt(bias, "bias", (torch.float32, torch.bfloat16))
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
    if out is not None:
        increment_version(out)  # the library wrote it through a raw pointer
    return Y


@dataclass
class LinearOut:
    """One linear of ``w4_linear_cached_rot_multi``: packed weights [N, K/2] with their row
    scales (and zero points), optional bias [N] and low-rank branch (t given), and the output
    (a new tensor unless ``out`` is given)."""
    packed: torch.Tensor
    row_scale: torch.Tensor
    zp: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None
    lowrank: Optional[LowRank] = None
    out_i32: bool = False
    out: Optional[torch.Tensor] = None


MULTI_MAX = 8


def w4_linear_cached_rot_multi(q, tok_scale, tok_rowsum, act_bits: int, outs, ws=None):
    """Several linears on the same codes from ``w4_rotate_quant_act`` (consecutive compatible
    pairs run as one launch for M > 64).  Returns the list of outputs Y_i [M, N_i]."""
    lib = load_library()
    if act_bits not in (4, 8):
        raise ValueError("act_bits must be 4 or 8, got %r" % (act_bits,))
    outs = list(outs)
    if not 1 <= len(outs) <= MULTI_MAX:
        raise ValueError("outs must hold 1..%d linears, got %d" % (MULTI_MAX, len(outs)))
    K = 2 * _matrix(outs[0].packed, "outs[0].packed")[1]
    M = _matrix(q, "q")[0]
    _shape(q, "q", (M, K) if act_bits == 8 else (M, K // 2))
    _shape(tok_scale, "tok_scale", (M,))
    _shape(tok_rowsum, "tok_rowsum", (M,))
    for i, o in enumerate(outs):
        N, Kh = _matrix(o.packed, "outs[%d].packed" % i)
        if 2 * Kh != K:
            raise ValueError("outs[%d].packed has K=%d, expected %d" % (i, 2 * Kh, K))
        _check_weights(o.packed, o.row_scale, o.zp, o.bias, N, K)
        if o.lowrank is not None and not o.out_i32:
            if o.lowrank.t is None:
                raise ValueError("outs[%d].lowrank must give t" % i)
            o.lowrank.check(M, N, K, need_t=True)
        if o.out is not None:
            _shape(o.out, "outs[%d].out" % i, (M, N))
    _dev(q, "q", (torch.int8,) if act_bits == 8 else (torch.uint8,))
    _dev(tok_scale, "tok_scale", (torch.float32,))
    _dev(tok_rowsum, "tok_rowsum", (torch.int32,))
    arr = (_LinearOutC * len(outs))()
    keep, Ys = [], []
    for i, o in enumerate(outs):
        _dev(o.packed, "packed", (torch.uint8,))
        _dev(o.row_scale, "row_scale", (torch.float32,))
        _opt(o.zp, "zp", (torch.uint8,))
        _opt(o.bias, "bias", (torch.float32, torch.bfloat16))
        N = o.packed.shape[0]
        Y = _y(M, N, o.out_i32, o.packed.device, o.out)
        Ys.append(Y)
        c = arr[i]
        c.packed, c.row_scale = o.packed.data_ptr(), o.row_scale.data_ptr()
        c.zp = o.zp.data_ptr() if o.zp is not None else None
        c.bias = o.bias.data_ptr() if o.bias is not None else None
        c.bias_dtype = _fdtype(o.bias) if o.bias is not None else W4_BF16
        if o.lowrank is not None and not o.out_i32:
            lrc = o.lowrank.as_c()
            keep.append(lrc)
            c.lr = ctypes.pointer(lrc)
        c.N, c.Y = N, Y.data_ptr()
        c.y_kind = W4_OUT_I32 if o.out_i32 else W4_OUT_BF16
    need = max(w4_workspace_bytes(M, o.packed.shape[0], K, act_bits, 0) for o in outs)
    ws = _ws(need, q.device, ws)
    _check(lib.w4_linear_cached_rot_multi(
        q.data_ptr(), tok_scale.data_ptr(), tok_rowsum.data_ptr(), act_bits, M, K, len(outs), arr,
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream(q.device)))
    for o in outs:
        if o.out is not None:
            increment_version(o.out)  # the library wrote it through a raw pointer
    return Ys


def w4_linear(X, g: int, act_bits: int, packed, row_scale, zp=None, bias=None,
              lowrank: Optional[LowRank] = None, out_i32: bool = False, out=None, ws=None):
    """The whole layer on X [M, K]: rotate + quantize, GEMM, fused dequant.  Returns Y [M, N]."""
    lib = load_library()
    M, K = _matrix(X, "X")
    N = _matrix(packed, "packed")[0]
    _check_weights(packed, row_scale, zp, bias, N, K)
    if lowrank is not None:
        lowrank.check(M, N, K, need_t=not out_i32)
    _dev(X, "X", (torch.float32, torch.bfloat16))
    _dev(packed, "packed", (torch.uint8,))
    _dev(row_scale, "row_scale", (torch.float32,))
    _opt(zp, "zp", (torch.uint8,))
    _opt(bias, "bias", (torch.float32, torch.bfloat16))
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
    if out is not None:
        increment_version(out)  # the library wrote it through a raw pointer
    return Y


def w4_noalloc_scratch_bytes() -> int:
    return int(load_library().w4_noalloc_scratch_bytes())


def w4_linear_noalloc(X, g: int, act_bits: int, packed, row_scale, zp=None, bias=None,
                      lowrank: Optional[LowRank] = None, out_i32: bool = False, out=None):
    """w4_linear without a workspace: the library's per-device scratch array holds the codes.

    For callers that cannot allocate device memory inside the call (graph capture, serving
    loops): pass ``out`` to keep torch from allocating the output as well.  Calls that overlap
    on one GPU share the scratch and must be ordered by the caller."""
    lib = load_library()
    M, K = _matrix(X, "X")
    N = _matrix(packed, "packed")[0]
    _check_weights(packed, row_scale, zp, bias, N, K)
    if lowrank is not None:
        lowrank.check(M, N, K, need_t=not out_i32)
    _dev(X, "X", (torch.float32, torch.bfloat16))
    _dev(packed, "packed", (torch.uint8,))
    _dev(row_scale, "row_scale", (torch.float32,))
    _opt(zp, "zp", (torch.uint8,))
    _opt(bias, "bias", (torch.float32, torch.bfloat16))
    Y = _y(M, N, out_i32, X.device, out)
    lrc = lowrank.as_c() if lowrank is not None else None
    _check(lib.w4_linear_noalloc(
        X.data_ptr(), _fdtype(X), M, K, g, act_bits, packed.data_ptr(), row_scale.data_ptr(),
        zp.data_ptr() if zp is not None else None, bias.data_ptr() if bias is not None else None,
        _fdtype(bias) if bias is not None else W4_BF16,
        ctypes.byref(lrc) if lrc is not None else None, N, Y.data_ptr(),
        W4_OUT_I32 if out_i32 else W4_OUT_BF16, _stream(X.device)))
    if out is not None:
        increment_version(out)  # the library wrote it through a raw pointer
    return Y


# ------------------------------------------------------------------ grouped-scale weight format
def w4_grouped_workspace_bytes(M, N, K, act_bits, gw, r=0) -> int:
    return int(load_library().w4_grouped_workspace_bytes(M, N, K, act_bits, gw, r))


def w4_linear_grouped_workspace_bytes(M, N, K, act_bits, gw, r=0) -> int:
    return int(load_library().w4_linear_grouped_workspace_bytes(M, N, K, act_bits, gw, r))


def w4_pack_weights_grouped(W: torch.Tensor, g: int, gw: int):
    """Rotate (g = 0: not at all), quantize per (row, run of gw inputs) and pack W [N, K].

    Returns (packed uint8 [N, K/2], group_scale fp16 [N, K/gw])."""
    lib = load_library()
    N, K = _matrix(W, "W")
    if gw <= 0 or K % gw:
        raise ValueError("K=%d is not a multiple of gw=%r" % (K, gw))
    _dev(W, "W", (torch.float32, torch.bfloat16))
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scale = torch.empty((N, K // gw), dtype=torch.float16, device=W.device)
    _check(lib.w4_pack_weights_grouped(W.data_ptr(), _fdtype(W), N, K, g, gw, packed.data_ptr(),
                                       scale.data_ptr(), _stream(W.device)))
    return packed, scale


def _check_grouped(packed, group_scale, bias, N, K):
    _shape(packed, "packed", (N, K // 2))
    gw = K // int(_matrix(group_scale, "group_scale")[1]) if group_scale.shape[1] else 0
    _shape(group_scale, "group_scale", (N, K // gw if gw else -1))
    if gw * group_scale.shape[1] != K:
        raise ValueError("group_scale width %d does not divide K=%d" % (group_scale.shape[1], K))
    _shape(bias, "bias", (N,))
    return gw


def w4_linear_cached_rot_grouped(q, tok_scale, act_bits: int, packed, group_scale, bias=None,
                                 lowrank: Optional[LowRank] = None, out_i32: bool = False, out=None, ws=None):
    """Grouped-scale GEMM + dequant on codes from ``w4_rotate_quant_act``.  Returns Y [M, N]."""
    lib = load_library()
    if act_bits not in (4, 8):
        raise ValueError("act_bits must be 4 or 8, got %r" % (act_bits,))
    N, Kh = _matrix(packed, "packed")
    K = 2 * Kh
    M = _matrix(q, "q")[0]
    _shape(q, "q", (M, K) if act_bits == 8 else (M, K // 2))
    _shape(tok_scale, "tok_scale", (M,))
    gw = _check_grouped(packed, group_scale, bias, N, K)
    if lowrank is not None:
        lowrank.check(M, N, K, need_t=not out_i32)
    _dev(q, "q", (torch.int8,) if act_bits == 8 else (torch.uint8,))
    _dev(tok_scale, "tok_scale", (torch.float32,))
    _dev(packed, "packed", (torch.uint8,))
    _dev(group_scale, "group_scale", (torch.float16,))
    _opt(bias, "bias", (torch.float32, torch.bfloat16))
    Y = _y(M, N, out_i32, packed.device, out)
    lrc = lowrank.as_c() if lowrank is not None else None
    r = lowrank.r if (lowrank is not None and lowrank.t is None and not out_i32) else 0
    ws = _ws(w4_grouped_workspace_bytes(M, N, K, act_bits, gw, r), packed.device, ws)
    _check(lib.w4_linear_cached_rot_grouped(
        q.data_ptr(), tok_scale.data_ptr(), act_bits, packed.data_ptr(), group_scale.data_ptr(), gw,
        bias.data_ptr() if bias is not None else None, _fdtype(bias) if bias is not None else W4_BF16,
        ctypes.byref(lrc) if lrc is not None else None, M, N, K, Y.data_ptr(),
        W4_OUT_I32 if out_i32 else W4_OUT_BF16,
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream(packed.device)))
    if out is not None:
        increment_version(out)
    return Y


def w4_linear_grouped(X, g: int, act_bits: int, packed, group_scale, bias=None,
                      lowrank: Optional[LowRank] = None, out_i32: bool = False, out=None, ws=None):
    """The layer on the grouped-scale format: W4A8 / W4A4 (rotation g > 0) or W4A16 (g = 0,
    act_bits = 16, bf16 X).  Returns Y [M, N]."""
    lib = load_library()
    M, K = _matrix(X, "X")
    N = _matrix(packed, "packed")[0]
    gw = _check_grouped(packed, group_scale, bias, N, K)
    if lowrank is not None:
        lowrank.check(M, N, K, need_t=not out_i32)
    _dev(X, "X", (torch.float32, torch.bfloat16))
    _dev(packed, "packed", (torch.uint8,))
    _dev(group_scale, "group_scale", (torch.float16,))
    _opt(bias, "bias", (torch.float32, torch.bfloat16))
    Y = _y(M, N, out_i32, X.device, out)
    lrc = lowrank.as_c() if lowrank is not None else None
    r = lowrank.r if (lowrank is not None and lowrank.t is None and not out_i32) else 0
    ws = _ws(w4_linear_grouped_workspace_bytes(M, N, K, act_bits, gw, r), X.device, ws)
    _check(lib.w4_linear_grouped(
        X.data_ptr(), _fdtype(X), M, K, g, act_bits, packed.data_ptr(), group_scale.data_ptr(), gw,
        bias.data_ptr() if bias is not None else None, _fdtype(bias) if bias is not None else W4_BF16,
        ctypes.byref(lrc) if lrc is not None else None, N, Y.data_ptr(),
        W4_OUT_I32 if out_i32 else W4_OUT_BF16,
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream(X.device)))
    if out is not None:
        increment_version(out)
    return Y


def w4_lowrank_down(x: torch.Tensor, l1: torch.Tensor) -> torch.Tensor:
    """t = x . L1 (f32 [M, r]) for a low-rank branch, shareable by linears reading x.

    ``l1`` is L1 transposed, bf16 [r, K] (rank-major, like a LoRA down weight)."""
    lib = load_library()
    M, K = _matrix(x, "x")
    r = _matrix(l1, "l1")[0]
    _shape(l1, "l1", (r, K))
    _dev(x, "x", (torch.bfloat16,))
    _dev(l1, "l1", (torch.bfloat16,))
    t = torch.empty((M, r), dtype=torch.float32, device=x.device)
    _check(lib.w4_lowrank_down(x.data_ptr(), l1.data_ptr(), M, K, r, t.data_ptr(), _stream(x.device)))
    return t


class RotationCache:
    """Rotated + quantized activations shared by linears that read the same input.

    stable-diffusion.cpp PR #2010, "Summary": the activation rotation / quantize is
    shared and cached per (input, group size).  The key is the tensor's identity
    (storage pointer, offset, shape, strides, dtype), torch's in-place version counter,
    the current stream, g and act_bits; the entry keeps a reference to the input, so its
    storage cannot be freed and reused while cached.  Scope it to one block / forward and
    ``clear()`` it.

    The stream is part of the key because the cached codes are ordered only on the stream
    that produced them: a lookup from another stream recomputes instead of reading codes
    with no ordering against their producer.  The version counter sees torch's in-place
    ops and the ``out=`` buffers of this package's linears (they bump it); a tensor written
    through some other raw pointer must be bumped by its writer
    (``torch.autograd.graph.increment_version``) or the cache cleared."""

    def __init__(self):
        self._d = {}
        self.hits = 0
        self.misses = 0

    @staticmethod
    def _stream_of(X: torch.Tensor) -> int:
        return torch.cuda.current_stream(X.device).cuda_stream if X.is_cuda else 0

    @classmethod
    def _key(cls, X: torch.Tensor, g: int, act_bits: int):
        return (X.data_ptr(), X.storage_offset(), tuple(X.shape), tuple(X.stride()), X.dtype,
                X._version, cls._stream_of(X), g, act_bits)

    def get(self, X: torch.Tensor, g: int, act_bits: int, l1: Optional[torch.Tensor] = None):
        """(q, tok_scale, tok_rowsum) for X, computed on a miss.  With ``l1`` (bf16 [r, K], the
        stacked L1 factors of every linear that reads X) the entry also holds t = X . L1 from
        the same pass, returned as a fourth value; give the same l1 on every lookup of X."""
        k = self._key(X, g, act_bits) + ((l1.data_ptr(), tuple(l1.shape), l1._version) if l1 is not None else ())
        hit = self._d.get(k)
        if hit is not None:
            self.hits += 1
            return hit[1]
        self.misses += 1
        if l1 is not None:
            val = w4_rotate_quant_act_lowrank(X, g, act_bits, l1)
            self._d[k] = ((X, l1), val)
        else:
            val = w4_rotate_quant_act(X, g, act_bits)
            self._d[k] = (X, val)
        return val

    def clear(self):
        self._d.clear()

    def __len__(self):
        return len(self._d)
