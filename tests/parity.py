"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Bars:
  * integer work (packed bytes, accumulators on given codes, row sums): bit-exact;
  * quantized codes: equal, except that a code may differ by exactly 1 where the
    oracle's fp64 pre-round value lies within 1e-6 of a rounding tie;
  * scales: bit-equal, except where fp64 absmax/qmax lies within 2^-40 (relative) of
    an fp32 rounding midpoint (the two sides round the same fp64 value; the only
    freedom is the last bit of that value);
  * bf16 outputs: relative Frobenius error <= 5e-3 against the oracle's fp64 output.
    (bf16 rounding alone contributes ~1.1e-3; the fp32 epilogue ~1e-7.)
"""
import numpy as np
import torch

TIE_WINDOW = 1e-6
FROB_TOL = 5e-3


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def check_codes(gpu: np.ndarray, ref: np.ndarray, pre: np.ndarray, what: str) -> int:
    """Codes must match except +-1 where the oracle's pre-round value is within 1e-6 of a tie.
    Returns the number of (allowed) tie mismatches."""
    gpu = gpu.astype(np.int64)
    ref = ref.astype(np.int64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    diff = gpu != ref
    n = int(diff.sum())
    if n:
        d = np.abs(gpu[diff] - ref[diff])
        frac = np.abs(pre[diff] - np.floor(pre[diff]) - 0.5)
        bad = (d != 1) | (frac > TIE_WINDOW)
        if bad.any():
            idx = np.argwhere(diff)[bad][:5]
            raise AssertionError("%s: %d code mismatches outside the tie window, e.g. at %s "
                                 "(gpu %s, oracle %s, pre %s)" % (
                                     what, int(bad.sum()), idx.tolist(), gpu[tuple(idx.T)].tolist(),
                                     ref[tuple(idx.T)].tolist(), pre[tuple(idx.T)].tolist()))
    return n


def _near_f32_midpoint(t: float, rel=2.0 ** -40) -> bool:
    s = np.float32(t)
    for nb in (np.nextafter(s, np.float32(np.inf)), np.nextafter(s, np.float32(-np.inf))):
        mid = (float(s) + float(nb)) / 2
        if abs(t - mid) <= rel * abs(t):
            return True
    return False


def check_scales(gpu: np.ndarray, ref: np.ndarray, unrounded: np.ndarray, what: str) -> np.ndarray:
    """Bit-equal fp32 scales, except rows whose fp64 value sits on an fp32 midpoint.
    Returns the boolean mask of rows whose scales agree."""
    gpu = np.asarray(gpu, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float32)
    eq = gpu.view(np.uint32) == ref.view(np.uint32)
    for i in np.flatnonzero(~eq):
        assert _near_f32_midpoint(float(unrounded[i])), \
            "%s: scale %d differs (gpu %r, oracle %r)" % (what, i, gpu[i], ref[i])
    return eq


def rel_frob(y: torch.Tensor, ref64: np.ndarray) -> float:
    yv = np_(y.float()).astype(np.float64)
    den = np.linalg.norm(ref64)
    return float(np.linalg.norm(yv - ref64) / (den if den > 0 else 1.0))


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    """Seeded sample of n rows that always includes the first and the last row."""
    if M <= n:
        return np.arange(M)
    r = np.random.Generator(np.random.PCG64(seed))
    rows = set(r.choice(M, size=n - 2, replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows))
