"""Plain fp64 / int64 statement of the ConvRot INT4 weight-quantized linear.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources, cited by page title and section:
  [CRUSH]  "ComfyUI-INT-Crush" README: sections "Inference / INT4" (unpack
           INT4 -> INT8, INT8 GEMM with fused dequant; fused ConvRot path =
           Hadamard rotation + activation quantization + INT8 GEMM; W4A8 =
           unpack, dynamic activation quantization, fused GEMM + dequant),
           "Inference / INT8" (dynamic per-token INT8 activation quantization),
           "LoRA" (residuals live in unrotated activation space),
           "Weight Format" (uint8 weights, two 4-bit values per byte, with
           scales) and "Forward Pass" (rotate, pad, quantize + GEMM, then the
           SVD low-rank residual L1/L2).
  [SDCPP]  "feat: packed int4 convrot model loading and dispatch #2010"
           (stable-diffusion.cpp): "Summary" (formats convrot_w4a4 and
           asym_w4a8_int8, packed nibbles passed raw with row scales, rotation
           and activation quantization cached per (input, group size)),
           "Backend notes" (group sizes 64 and 256), "Verification" (W4A4 is
           checked bitwise against a CPU oracle) and the shape report in the
           discussion (a packed weight's input dimension is half the logical
           one, i.e. the nibbles are packed along K).
  [TINT4]  "TINT4 v1.2 - torchao INT4 for ComfyUI": the quantized linear keeps
           codes, a scale and a zero point (v1.1 section 5).

Where the pages leave a step open, the reading taken here is stated at the
function (Hadamard normalisation, rounding rule, scale formulas, nibble order,
zero handling); each such reading is also listed with the design notes.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

from . import _native

__all__ = [
    "QMAX", "to_f64", "hadamard", "rotate", "quant_weights_sym", "quant_weights_asym",
    "quant_act", "pack_nibbles", "unpack_nibbles", "gemm_i64", "epilogue", "bf16_rne",
    "bf16_bits_to_f64", "lowrank", "pack_weights", "rotate_quant_act", "weight_operand",
    "linear_from_codes", "linear", "gelu_bf16", "num_threads", "f16_rne", "quant_weights_grouped",
    "gemm_i64_groups", "epilogue_grouped", "dequant_grouped", "pack_weights_grouped", "linear_grouped",
]

# Largest code magnitude for per-token activation codes, by bit width.
QMAX = {8: 127, 4: 7}


# --------------------------------------------------------------------------- inputs
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the 16 bits are the top half of an fp32."""
    u = bits.astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(t) -> np.ndarray:
    """Exact fp64 copy of a bf16 / fp32 / fp64 tensor or array (widening only)."""
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu").contiguous()
        if t.dtype == torch.bfloat16:
            return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
        if t.dtype in (torch.float32, torch.float64):
            return t.numpy().astype(np.float64)
        raise TypeError("unsupported dtype %s" % t.dtype)
    a = np.asarray(t)
    if a.dtype not in (np.float32, np.float64):
        raise TypeError("unsupported dtype %s" % a.dtype)
    return a.astype(np.float64)


# --------------------------------------------------------------------------- rotation
def _popcount(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.int64)
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a = a >> 1
    return c


@functools.lru_cache(maxsize=8)
def _hadamard_cached(g: int) -> np.ndarray:
    if g < 1 or g & (g - 1):
        raise ValueError("g must be a power of two")
    i = np.arange(g, dtype=np.int64)
    H = np.where(_popcount(i[:, None] & i[None, :]) % 2 == 0, 1, -1).astype(np.int64)
    H.setflags(write=False)
    return H


def hadamard(g: int) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard matrix H_g[i, j] = (-1)^popcount(i & j).

    [CRUSH] "Inference / INT4" names a Hadamard rotation of the activations in
    blocks of rot_size; the pages never print the matrix.  Reading: the
    Sylvester (Walsh) ordering, no random sign flips, the same matrix for
    activations and weights, so the rotation cancels in the product.  (Built once per g and
    kept; the caller gets a fresh copy.)"""
    return _hadamard_cached(int(g)).copy()


def rotate(A: np.ndarray, g: int) -> np.ndarray:
    """A . blockdiag(H_g / sqrt(g)) along the last axis, as one explicit g x g
    matrix multiply per contiguous group of g columns.

    [CRUSH] "Forward Pass" step 2 rotates the activations; [SDCPP] "Summary"
    and "Backend notes" key the rotation by group size (64 and 256 verified);
    [CRUSH] "Nodes" lists the rotation sizes 0/16/64/256/1024/4096.
    Reading: contiguous groups [j*g, (j+1)*g) along K; K % g == 0 (padding to
    in_features is the caller's step 3); normalised by 1/sqrt(g), which is a
    power of two for g = 4^n, so the scaling is exact.  g = 0 is "no rotation"
    (the W4A16 path of [CRUSH] "Inference / INT4"): A is returned unchanged."""
    A = np.asarray(A, dtype=np.float64)
    if g == 0:
        return A.copy()
    R, K = A.shape
    if K % g:
        raise ValueError("K=%d is not a multiple of g=%d" % (K, g))
    Hn = hadamard(g).astype(np.float64) / np.sqrt(np.float64(g))
    return (A.reshape(R, K // g, g) @ Hn).reshape(R, K)


# --------------------------------------------------------------------------- quantizers
def _safe_div(v: np.ndarray, s64: np.ndarray) -> np.ndarray:
    """v / s row-wise in fp64; rows whose scale is 0 give 0 (never divided)."""
    nz = s64 > 0
    out = np.zeros_like(v)
    out[nz] = v[nz] / s64[nz][:, None]
    return out


def quant_weights_sym(Wr: np.ndarray):
    """Per-output-row symmetric int4 codes of rotated weights.

    [TINT4] v1.1 section 5 and [CRUSH] "Weight Format": 4-bit codes with a
    scale per output row.  Reading: s = fp32(max|w'| / 7) (division in fp64,
    one rounding to fp32); c = clamp(rint(w' / s), -8, 7) with the division in
    fp64 by the stored fp32 scale and round-half-to-even; a zero row gets s = 0
    and codes 0.  Returns (codes int8 [N, K], scale f32 [N], pre-round values)."""
    amax = np.max(np.abs(Wr), axis=1)
    s = (amax / 7.0).astype(np.float32)
    pre = _safe_div(Wr, s.astype(np.float64))
    c = np.clip(np.rint(pre), -8, 7).astype(np.int8)
    return c, s, pre


def quant_weights_asym(Wr: np.ndarray):
    """Per-output-row asymmetric (unsigned) int4 codes with a zero point.

    [SDCPP] "Summary" names the asymmetric W4A8 format; [TINT4] keeps
    codes, scale and zero point.  Reading: lo = min(min w', 0),
    hi = max(max w', 0), s = fp32((hi - lo) / 15), z = clamp(-rint(lo / s), 0, 15),
    c = clamp(rint(w' / s) + z, 0, 15): round first, then add z.  A zero row
    gets s = 0, z = 0, codes 0.  Returns (codes uint8 [N, K], scale f32 [N],
    zp uint8 [N], pre-round values of w'/s, pre-round values of -lo/s)."""
    lo = np.minimum(Wr.min(axis=1), 0.0)
    hi = np.maximum(Wr.max(axis=1), 0.0)
    s = ((hi - lo) / 15.0).astype(np.float32)
    s64 = s.astype(np.float64)
    zpre = np.zeros_like(lo)
    nz = s64 > 0
    zpre[nz] = -lo[nz] / s64[nz]
    z = np.clip(np.rint(zpre), 0, 15).astype(np.int64)
    pre = _safe_div(Wr, s64)
    c = np.clip(np.rint(pre) + z[:, None], 0, 15).astype(np.uint8)
    return c, s, z.astype(np.uint8), pre, zpre


def quant_act(Xr: np.ndarray, bits: int):
    """Per-token dynamic symmetric activation codes.

    [CRUSH] "Inference / INT8" (dynamic per-token INT8 quantization) and
    "Inference / INT4" (dynamic activation quantization before the GEMM); the
    W4A4 format of [SDCPP] "Summary" uses 4-bit activations.  Reading:
    s = fp32(max|x'| / qmax), qmax = 127 (8 bits) or 7 (4 bits);
    q = clamp(rint(x' / s), -qmax - 1, qmax), division in fp64 by the stored
    fp32 scale, round-half-to-even; an all-zero token gets s = 0, codes 0.
    Returns (q int8 [M, K], scale f32 [M], rowsum int64 [M], pre-round values)."""
    qmax = QMAX[bits]
    amax = np.max(np.abs(Xr), axis=1) if Xr.shape[1] else np.zeros(Xr.shape[0])
    s = (amax / float(qmax)).astype(np.float32)
    pre = _safe_div(Xr, s.astype(np.float64))
    q = np.clip(np.rint(pre), -qmax - 1, qmax).astype(np.int8)
    return q, s, q.astype(np.int64).sum(axis=1), pre


def f16_rne(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp16, one round-to-nearest-even (NumPy's double -> half conversion rounds the
    fp64 value directly, with no intermediate fp32 step; pinned against exact rationals)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def quant_weights_grouped(Wr: np.ndarray, gw: int):
    """Symmetric int4 codes with one fp16 scale per output row and group of gw inputs.

    [CRUSH] "Weight Format": INT4 weights are uint8 (two per byte) plus weight_scale fp16
    [out, num_groups].  Reading: groups are contiguous runs of gw along K (num_groups =
    K / gw); s = fp16(max|w'| / 7) over the group (fp64 division, one rounding to fp16);
    c = clamp(rint(w' / s), -8, 7) with the division in fp64 by the stored fp16 scale.  A
    group whose scale is 0 (all zero, or below fp16's smallest subnormal after rounding) gets
    codes 0; a scale that overflows fp16 is rejected.  Returns (codes int8 [N, K],
    scale f16 [N, K/gw], pre-round values)."""
    N, K = Wr.shape
    if gw < 1 or K % gw:
        raise ValueError("K=%d is not a multiple of gw=%d" % (K, gw))
    G = Wr.reshape(N, K // gw, gw)
    amax = np.max(np.abs(G), axis=2)
    s = f16_rne(amax / 7.0)
    if not np.all(np.isfinite(s)):
        raise OverflowError("group scale exceeds fp16")
    s64 = s.astype(np.float64)
    pre = np.zeros_like(G)
    nz = s64 > 0
    pre[nz] = G[nz] / s64[nz][:, None]
    c = np.clip(np.rint(pre), -8, 7).astype(np.int8)
    return c.reshape(N, K), s, pre.reshape(N, K)


# --------------------------------------------------------------------------- nibble codec
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte along K, low nibble = even k.

    [CRUSH] "Weight Format": uint8, 2 values per byte; [SDCPP] discussion:
    the packed input dimension is half the logical one (packed along K).
    Reading: byte j of a row = (c[2j] & 15) | (c[2j+1] & 15) << 4; signed codes
    are stored as 4-bit two's complement."""
    c = np.asarray(codes).astype(np.int64)
    if c.shape[-1] % 2:
        raise ValueError("odd K")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, signed: bool) -> np.ndarray:
    """Inverse of pack_nibbles: int16 codes, K = 2 * packed width."""
    p = np.asarray(packed).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    if signed:
        out = np.where(out >= 8, out - 16, out).astype(np.int16)
    return out


# --------------------------------------------------------------------------- GEMM + epilogue
def gemm_i64(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * w[n, k] in int64 (plain C triple loop).

    [CRUSH] "Forward Pass" step 5 and "Inference / INT4": integer GEMM of
    activation codes with the unpacked weight codes."""
    q8 = np.ascontiguousarray(q, dtype=np.int8)
    w8 = np.ascontiguousarray(w, dtype=np.int8)
    if not (np.array_equal(q8, q) and np.array_equal(w8, w)):
        raise ValueError("codes out of int8 range")
    M, K = q8.shape
    N, K2 = w8.shape
    if K != K2:
        raise ValueError("K mismatch")
    acc = np.zeros((M, N), dtype=np.int64)
    rc = _native.lib().oracle_gemm_i64(q8.ctypes.data, w8.ctypes.data, M, N, K, acc.ctypes.data)
    if rc:
        raise RuntimeError("oracle_gemm_i64 failed")
    return acc


def num_threads() -> int:
    return int(_native.lib().oracle_num_threads())


def epilogue(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray, bias=None, lr=None) -> np.ndarray:
    """y = acc * s_x[m] * s_w[n] + lr[m, n] + bias[n], all in fp64.

    [CRUSH] "Inference / INT4": INT8 GEMM with fused dequant; "Forward Pass"
    step 6 adds the low-rank residual after the GEMM.  Reading: the low-rank
    term is added before the bias."""
    y = acc.astype(np.float64) * s_x.astype(np.float64)[:, None] * s_w.astype(np.float64)[None, :]
    if lr is not None:
        y = y + lr
    if bias is not None:
        y = y + to_f64(bias)[None, :]
    return y


def gemm_i64_groups(q: np.ndarray, w: np.ndarray, gw: int) -> np.ndarray:
    """acc_j[m, n] = sum over k in group j of q[m, k] * w[n, k]: the int64 GEMM of each
    contiguous group of gw inputs.  Returns int64 [K / gw, M, N]."""
    K = q.shape[1]
    if K % gw:
        raise ValueError("K=%d is not a multiple of gw=%d" % (K, gw))
    return np.stack([gemm_i64(np.ascontiguousarray(q[:, j:j + gw]), np.ascontiguousarray(w[:, j:j + gw]))
                     for j in range(0, K, gw)])


def epilogue_grouped(acc_g: np.ndarray, s_x: np.ndarray, s_wg: np.ndarray, bias=None, lr=None) -> np.ndarray:
    """y[m, n] = s_x[m] * sum_j s_w[n, j] * acc_j[m, n] + lr[m, n] + bias[n], in fp64.

    With one weight scale per group the group partial sums are scaled before they are added
    ([CRUSH] "Weight Format" scales [out, num_groups]; "Inference / INT4" fused dequant)."""
    sw = s_wg.astype(np.float64)                       # [N, G]
    y = np.einsum("jmn,nj->mn", acc_g.astype(np.float64), sw) * s_x.astype(np.float64)[:, None]
    if lr is not None:
        y = y + lr
    if bias is not None:
        y = y + to_f64(bias)[None, :]
    return y


def bf16_rne(y: np.ndarray) -> torch.Tensor:
    """Round fp64 values once to bf16, nearest-even, by explicit quantum arithmetic.

    A finite x with |x| >= 2^-126 has bf16 quantum 2^(e - 8) where x = m * 2^e,
    0.5 <= |m| < 1 (8 significant bits); below that the subnormal quantum 2^-133
    applies.  x / quantum is exact (a power of two), rint rounds it half-to-even,
    and the result times the quantum is a bf16 value (or overflows to inf)."""
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.float64)
    fin = np.isfinite(y)
    yf = y[fin]
    _, e = np.frexp(yf)
    e = np.maximum(e, -125)  # |x| < 2^-126 -> subnormal quantum 2^-133
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(yf / quantum) * quantum
    r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
    out[fin] = r
    out[~fin] = y[~fin]
    f32 = out.astype(np.float32)  # exact: every value is a bf16 value
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)


def lowrank(X, L1, L2) -> np.ndarray:
    """(X . L1) . L2 in fp64 with the unrotated activations.

    [CRUSH] "Forward Pass" step 6 (SVD low-rank residual from L1/L2 factors)
    and "LoRA" (residual branches read the unrotated activations)."""
    return (to_f64(X) @ to_f64(L1)) @ to_f64(L2)


def gelu_bf16(y: torch.Tensor) -> torch.Tensor:
    """Host glue between the MLP linears: erf GELU of bf16 values, in fp64, to bf16.

    Not part of the quantized linear; it only produces the next linear's input."""
    import scipy.special
    x = to_f64(y)
    return bf16_rne(0.5 * x * (1.0 + scipy.special.erf(x / np.sqrt(2.0))))


def dequant_grouped(packed: np.ndarray, s_wg: np.ndarray, gw: int) -> np.ndarray:
    """W_hat[n, k] = s_w[n, k // gw] * c[n, k] in fp64 (exact: fp16 times a small integer)."""
    c = unpack_nibbles(packed, signed=True).astype(np.float64)
    N, K = c.shape
    return (c.reshape(N, K // gw, gw) * s_wg.astype(np.float64)[:, :, None]).reshape(N, K)


# --------------------------------------------------------------------------- pipeline
def pack_weights(W, g: int, asym: bool) -> dict:
    """Offline weight step: rotate rows, quantize per row, pack two nibbles per byte."""
    Wr = rotate(to_f64(W), g)
    if asym:
        c, s, z, pre, zpre = quant_weights_asym(Wr)
        return {"packed": pack_nibbles(c), "scale": s, "zp": z, "codes": c.astype(np.int16),
                "pre": pre, "zpre": zpre, "rotated": Wr}
    c, s, pre = quant_weights_sym(Wr)
    return {"packed": pack_nibbles(c), "scale": s, "zp": None, "codes": c.astype(np.int16),
            "pre": pre, "rotated": Wr}


def pack_weights_grouped(W, g: int, gw: int) -> dict:
    """Offline step of the grouped-scale format: rotate rows (g = 0: none), quantize per
    (row, group of gw) with fp16 scales, pack two nibbles per byte."""
    Wr = rotate(to_f64(W), g)
    c, s, pre = quant_weights_grouped(Wr, gw)
    return {"packed": pack_nibbles(c), "scale": s, "codes": c.astype(np.int16), "pre": pre, "rotated": Wr,
            "gw": gw}


def rotate_quant_act(X, g: int, bits: int) -> dict:
    """Activation step: rotate each token, quantize per token (plus 4-bit packing)."""
    Xr = rotate(to_f64(X), g)
    q, s, rowsum, pre = quant_act(Xr, bits)
    out = {"q": q, "scale": s, "rowsum": rowsum, "pre": pre, "rotated": Xr}
    if bits == 4:
        out["packed"] = pack_nibbles(q)
    return out


def weight_operand(packed: np.ndarray, zp, asym: bool) -> np.ndarray:
    """Unpack the stored bytes again and take the zero point off: c - z (int8 range)."""
    c = unpack_nibbles(packed, signed=not asym).astype(np.int16)
    if asym:
        c = c - np.asarray(zp).astype(np.int16)[:, None]
    return c


def linear_from_codes(q, s_x, packed, s_w, zp, asym, bias=None, lr=None) -> dict:
    """Integer GEMM on given codes, then the fp64 epilogue and one bf16 rounding."""
    acc = gemm_i64(q, weight_operand(packed, zp, asym))
    if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
        raise OverflowError("accumulator exceeds int32")
    y64 = epilogue(acc, s_x, s_w, bias, lr)
    return {"acc": acc, "y64": y64, "y": bf16_rne(y64)}


def linear(X, W, g: int, act_bits: int, asym: bool, bias=None, L1=None, L2=None) -> dict:
    """The whole layer: pack W, rotate + quantize X, integer GEMM, dequant epilogue."""
    pw = pack_weights(W, g, asym)
    qa = rotate_quant_act(X, g, act_bits)
    lr = lowrank(X, L1, L2) if L1 is not None else None
    out = linear_from_codes(qa["q"], qa["scale"], pw["packed"], pw["scale"], pw["zp"], asym,
                            bias, lr)
    out.update({"w": pw, "a": qa, "lr": lr})
    return out


def linear_grouped(X, W, g: int, gw: int, act_bits: int, bias=None, L1=None, L2=None) -> dict:
    """The layer with grouped fp16 weight scales.

    act_bits 8 / 4: rotate + quantize X per token (g > 0), int64 GEMM per weight group,
    grouped fp64 epilogue.  act_bits 16 (W4A16, [CRUSH] "Inference / INT4", Triton backend:
    rot_size 0 unpacks INT4 to a float matrix for a plain GEMM): g must be 0; y = X . W_hat^T
    in fp64 with W_hat the dequantized weights.  Then lr and bias, one bf16 rounding."""
    pw = pack_weights_grouped(W, g, gw)
    lr = lowrank(X, L1, L2) if L1 is not None else None
    if act_bits == 16:
        if g != 0:
            raise ValueError("W4A16 takes unrotated weights (g = 0)")
        y64 = to_f64(X) @ dequant_grouped(pw["packed"], pw["scale"], gw).T
        if lr is not None:
            y64 = y64 + lr
        if bias is not None:
            y64 = y64 + to_f64(bias)[None, :]
        return {"y64": y64, "y": bf16_rne(y64), "w": pw, "lr": lr}
    if g == 0:
        raise ValueError("integer activations are rotated (g > 0)")
    qa = rotate_quant_act(X, g, act_bits)
    w = weight_operand(pw["packed"], None, False)
    acc_g = gemm_i64_groups(qa["q"], w, gw)
    acc = acc_g.sum(axis=0)
    if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
        raise OverflowError("accumulator exceeds int32")
    y64 = epilogue_grouped(acc_g, qa["scale"], pw["scale"], bias, lr)
    return {"acc": acc, "acc_groups": acc_g, "y64": y64, "y": bf16_rne(y64), "w": pw, "a": qa, "lr": lr}
