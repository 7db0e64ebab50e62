"""Seeded synthetic inputs for the INT4 weight-quantized (ConvRot) linear layer.

This module only draws random tensors. It holds none of the layer's arithmetic
(no rotation, no quantization, no GEMM), so both the HIP path and the CPU oracle
can be fed from it without sharing any of the method.

Workloads (shapes and value distributions follow the diffusion-transformer
linears that the ConvRot loader pages run: FLUX / Z-Image style DiT blocks with
hidden size 3072, MLP ratio 4, 4096 image tokens (64x64 latent patches) plus 512
text tokens, and text-encoder linears with hidden 4096):

* ``tiny``         X [16, 256] fp32 ~N(0,1), 4 fixed outlier channels x20,
                   W [256, 256] ~N(0, 0.02), bias ~N(0, 0.01); g = 64, W4A8 sym.
* ``attn_proj``    X [4096, 3072] bf16 ~N(0,1), 1% of channels x30,
                   W [3072, 3072] ~N(0, 0.02), bias ~N(0, 0.01); g = 256, W4A8 sym.
* ``mlp_pair``     X as attn_proj -> up W [12288, 3072] -> GELU (host glue)
                   -> down W [3072, 12288]; g = 256, W4A4 sym.
* ``small_m``      (K, N) in {(4096, 12288), (12288, 4096)}, M in {1, 4, 16, 64};
                   1% of K outlier channels x30; g = 256, W4A8 asym (zero point).
* ``double_block`` 20 blocks of {QKV 3072->9216, out 3072->3072, up 3072->12288,
                   down 12288->3072} at M = 4608, rank-32 low-rank side branch
                   L1 [K, 32] (stored rank-major, [32, K]), L2 [32, N] ~N(0, 0.01); g = 256, W4A8 sym.

"N(0, s)" means standard deviation s.  Values are drawn in fp32 from NumPy's
PCG64 and cast once to the stored dtype (bf16 casts round to nearest even), so
every consumer receives byte-identical tensors.  For the 20-block workload the
tensors are drawn on the device with torch's own generator instead (2.3 G
values would take minutes on the host); tests copy the parts they check back.

Seeds: seed = 1000 * workload + 10 * linear + tensor, with tensor ids
X = 0, W = 1, bias = 2, L1 = 3, L2 = 4, outlier-channel draw = 5; block b of the
20-block workload uses 4000 + 100 * b + 10 * linear + tensor.
"""
from __future__ import annotations

import numpy as np
import torch

T_X, T_W, T_BIAS, T_L1, T_L2, T_OUTLIER = 0, 1, 2, 3, 4, 5

WORKLOAD_IDS = {"tiny": 0, "attn_proj": 1, "mlp_pair": 2, "small_m": 3, "double_block": 4}

DIT_HIDDEN = 3072
DIT_MLP = 12288
DIT_QKV = 9216
DIT_TOKENS_IMG = 4096
DIT_TOKENS_TXT = 512
TE_HIDDEN = 4096
TE_WIDE = 12288
LOWRANK = 32


def _normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def outlier_channels(seed: int, K: int, n: int) -> np.ndarray:
    """Sorted, distinct channel indices (drawn once, used for every token)."""
    if n <= 0:
        return np.zeros((0,), dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(K, size=n, replace=False)).astype(np.int64)


def _to_torch(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype != torch.float32:
        t = t.to(dtype)  # fp32 -> bf16 round-to-nearest-even
    return t.to(device) if device is not None and str(device) != "cpu" else t


def activations(seed: int, M: int, K: int, *, n_outliers: int, outlier_scale: float,
                dtype=torch.bfloat16, device="cpu"):
    """X [M, K] ~N(0,1) with ``n_outliers`` fixed channels scaled by ``outlier_scale``.

    Returns (X, channels)."""
    x = _normal(seed, (M, K))
    ch = outlier_channels(seed + (T_OUTLIER - T_X), K, n_outliers)
    if ch.size:
        x[:, ch] *= np.float32(outlier_scale)
    return _to_torch(x, dtype, device), ch


def weights(seed: int, N: int, K: int, *, std: float = 0.02, dtype=torch.bfloat16, device="cpu"):
    return _to_torch(_normal(seed, (N, K), std), dtype, device)


def vector(seed: int, n: int, *, std: float, dtype=torch.bfloat16, device="cpu"):
    return _to_torch(_normal(seed, (n,), std), dtype, device)


def one_percent(K: int) -> int:
    return int(round(0.01 * K))


def linear_case(workload: str, linear: int, M: int, K: int, N: int, *, x_dtype=torch.bfloat16,
                w_dtype=torch.bfloat16, bias_dtype=torch.bfloat16, n_outliers=None,
                outlier_scale=30.0, rank: int = 0, device="cpu"):
    """One linear's inputs: dict(X, W, bias, outliers[, L1, L2])."""
    base = 1000 * WORKLOAD_IDS[workload] + 10 * linear
    if n_outliers is None:
        n_outliers = one_percent(K)
    X, ch = activations(base + T_X, M, K, n_outliers=n_outliers, outlier_scale=outlier_scale,
                        dtype=x_dtype, device=device)
    out = {
        "X": X,
        "W": weights(base + T_W, N, K, std=0.02, dtype=w_dtype, device=device),
        "bias": vector(base + T_BIAS, N, std=0.01, dtype=bias_dtype, device=device),
        "outliers": ch,
    }
    if rank:
        # L1 rank-major ([r, K], L1 transposed), as the low-rank calls take it
        out["L1"] = _to_torch(np.ascontiguousarray(_normal(base + T_L1, (K, rank), 0.01).T), torch.bfloat16, device)
        out["L2"] = _to_torch(_normal(base + T_L2, (rank, N), 0.01), torch.bfloat16, device)
    return out


def tiny(device="cpu"):
    """16 x 256 x 256, fp32 inputs, 4 outlier channels x20, g = 64, W4A8 symmetric."""
    return linear_case("tiny", 0, 16, 256, 256, x_dtype=torch.float32, w_dtype=torch.float32,
                       bias_dtype=torch.float32, n_outliers=4, outlier_scale=20.0, device=device)


def attn_proj(device="cpu", M: int = DIT_TOKENS_IMG):
    """DiT attention projection 3072 -> 3072 at 4096 tokens, g = 256, W4A8 symmetric."""
    return linear_case("attn_proj", 0, M, DIT_HIDDEN, DIT_HIDDEN, device=device)


def mlp_up(device="cpu", M: int = DIT_TOKENS_IMG):
    """DiT MLP up-projection 3072 -> 12288, X drawn as for attn_proj, g = 256, W4A4."""
    d = linear_case("mlp_pair", 0, M, DIT_HIDDEN, DIT_MLP, device=device)
    d["X"], d["outliers"] = attn_proj_input(device, M)
    return d


def attn_proj_input(device="cpu", M: int = DIT_TOKENS_IMG):
    base = 1000 * WORKLOAD_IDS["attn_proj"]
    return activations(base + T_X, M, DIT_HIDDEN, n_outliers=one_percent(DIT_HIDDEN),
                       outlier_scale=30.0, device=device)


def mlp_down_weights(device="cpu"):
    """Down-projection 12288 -> 3072 weights and bias (its input is GELU(up) from the caller)."""
    base = 1000 * WORKLOAD_IDS["mlp_pair"] + 10 * 1
    return {
        "W": weights(base + T_W, DIT_HIDDEN, DIT_MLP, device=device),
        "bias": vector(base + T_BIAS, DIT_HIDDEN, std=0.01, device=device),
    }


def small_m(M: int, K: int, N: int, device="cpu"):
    """HBM-bound text-encoder linear at M tokens, asymmetric W4A8, g = 256."""
    lin = {(TE_HIDDEN, TE_WIDE): 0, (TE_WIDE, TE_HIDDEN): 1}[(K, N)]
    return linear_case("small_m", lin, M, K, N, device=device)


DOUBLE_BLOCK_LINEARS = (
    ("qkv", DIT_HIDDEN, DIT_QKV),
    ("out", DIT_HIDDEN, DIT_HIDDEN),
    ("up", DIT_HIDDEN, DIT_MLP),
    ("down", DIT_MLP, DIT_HIDDEN),
)
DOUBLE_BLOCK_TOKENS = DIT_TOKENS_IMG + DIT_TOKENS_TXT
N_BLOCKS = 20


def _device_normal(seed: int, shape, std: float, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def double_block(b: int, device, M: int = DOUBLE_BLOCK_TOKENS, rank: int = LOWRANK):
    """Block ``b`` of the 20-block workload, drawn on ``device`` with torch's generator.

    Returns dict(x: block input [M, 3072], attn: out-proj input proxy [M, 3072],
    and per linear name: W [N, K], bias [N], L1 [r, K] (rank-major, L1 transposed), L2 [r, N])."""
    base = 4000 + 100 * b
    K = DIT_HIDDEN
    out = {}
    for which, off in (("x", 0), ("attn", 50)):
        x = _device_normal(base + off + T_X, (M, K), 1.0, device).float()
        ch = outlier_channels(base + off + T_OUTLIER, K, one_percent(K))
        if ch.size:
            idx = torch.as_tensor(ch, device=x.device)
            x[:, idx] *= 30.0
        out[which] = x.to(torch.bfloat16)
    for li, (name, k, n) in enumerate(DOUBLE_BLOCK_LINEARS):
        s = base + 10 * li
        out[name] = {
            "W": _device_normal(s + T_W, (n, k), 0.02, device),
            "bias": _device_normal(s + T_BIAS, (n,), 0.01, device),
            "L1": _device_normal(s + T_L1, (k, rank), 0.01, device).t().contiguous(),  # rank-major [r, K]
            "L2": _device_normal(s + T_L2, (rank, n), 0.01, device),
        }
    return out
