"""Full-size parity of the grouped-scale weight format on the workloads ``bench.py`` times for
it (needs an MI355X): W4A8 at 4096 x 3072 -> 3072 (g = 256, fp16 scale per row and 128
inputs), W4A16 at the same shape, and W4A16 at 1 and 16 tokens on the text-encoder shapes.

Inputs come from ``synth`` (the bench's own draws).  The oracle packs the weights and
rotates/quantizes the activations itself; the GPU's packing and codes are checked against
it, the integer sums of the oracle's codes are compared exactly over all M x N outputs, and
the bf16 output of the GPU's own packing and rotation (as in the timed path) is compared
with the oracle's fp64 result over every row and every 32-row block."""
import numpy as np
import pytest
import torch

import oracle
import synth
import int4_weight_quantized_block_amd as w4
from parity import check_codes, check_scales, np_, rel_frob, FROB_TOL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GW = 128  # bench.py's default group width


def say(*a):
    print(*a, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def near_f16_midpoint(v: float, rel=2.0 ** -40) -> bool:
    s = np.float16(v)
    for nb in (np.nextafter(s, np.float16(np.inf)), np.nextafter(s, np.float16(-np.inf))):
        mid = (float(s) + float(nb)) / 2
        if abs(v - mid) <= rel * abs(v):
            return True
    return False


def grouped_weights(W, g, tag):
    """Pack on the GPU and on the oracle; scales bit-equal except on fp16 midpoints, codes
    equal except within the tie window.  Returns (GPU packed, GPU scales, oracle dict)."""
    N, K = W.shape
    ref = oracle.pack_weights_grouped(W, g, GW)
    packed, gs = w4.w4_pack_weights_grouped(W.to(DEV), g, GW)
    sg, so = np_(gs), ref["scale"]
    diff = sg.view(np.uint16) != so.view(np.uint16)
    if diff.any():
        G = ref["rotated"].reshape(N, K // GW, GW)
        unr = np.abs(G).max(2) / 7.0
        for idx in np.argwhere(diff):
            assert near_f16_midpoint(float(unr[tuple(idx)])), (tag, idx)
    rows_ok = ~diff.any(1)
    codes = oracle.unpack_nibbles(np_(packed), signed=True)
    check_codes(codes[rows_ok], ref["codes"][rows_ok], ref["pre"][rows_ok], tag + " grouped w codes")
    return packed, gs, ref


def check_rows(y, y64, tag):
    err = rel_frob(y, y64)
    worst = max(rel_frob(y[m0:m0 + 32], y64[m0:m0 + 32]) for m0 in range(0, y64.shape[0], 32))
    say("  %s rel frob %.3e (worst 32-row block %.3e)" % (tag, err, worst))
    assert err <= FROB_TOL, (tag, err)
    assert worst <= 2 * FROB_TOL, (tag, worst)


def test_attn_proj_grouped_w4a8():
    d = synth.attn_proj()
    X, W, bias = d["X"], d["W"], d["bias"]
    M, K = X.shape
    N = W.shape[0]
    say("grouped W4A8 attn_proj M=%d K=%d N=%d g=256 gw=%d" % (M, K, N, GW))
    packed, gs, pw = grouped_weights(W, 256, "attn_proj_grouped")
    ra = oracle.rotate_quant_act(X, 256, 8)
    q, sx, _ = w4.w4_rotate_quant_act(X.to(DEV), 256, 8)
    amax64 = np.abs(ra["rotated"]).max(1) / oracle.QMAX[8]
    assert check_scales(np_(sx), ra["scale"], amax64, "tok_scale").all()
    check_codes(np_(q), ra["q"], ra["pre"], "act codes")
    # exact integer sums of the oracle's codes and weights, all M x N
    acc = w4.w4_linear_cached_rot_grouped(to_dev(ra["q"]), to_dev(ra["scale"]), 8, to_dev(pw["packed"]),
                                          to_dev(pw["scale"]), out_i32=True)
    w = oracle.weight_operand(pw["packed"], None, False)
    say("  oracle int64 GEMM over all %d x %d outputs" % (M, N))
    acc_o = oracle.gemm_i64(ra["q"], w)
    bad = np.argwhere(np_(acc).astype(np.int64) != acc_o)
    assert bad.size == 0, "accumulators: %d mismatches, first at %s" % (len(bad), bad[:4].tolist())
    del acc, acc_o
    # bf16 output of the GPU's rotation and packing, every row; the oracle's grouped fp64
    # epilogue in row chunks (the per-group sums of all rows would take GBs)
    y = w4.w4_linear_grouped(X.to(DEV), 256, 8, packed, gs, bias=bias.to(DEV))
    y64 = np.empty((M, N))
    for m0 in range(0, M, 512):
        acc_g = oracle.gemm_i64_groups(np.ascontiguousarray(ra["q"][m0:m0 + 512]), w, GW)
        y64[m0:m0 + 512] = oracle.epilogue_grouped(acc_g, ra["scale"][m0:m0 + 512], pw["scale"], bias)
    check_rows(y, y64, "attn_proj_grouped")


def w4a16_case(X, W, bias, tag):
    M, K = X.shape
    N = W.shape[0]
    say("W4A16 %s M=%d K=%d N=%d gw=%d" % (tag, M, K, N, GW))
    packed, gs, pw = grouped_weights(W, 0, tag)
    y = w4.w4_linear_grouped(X.to(DEV), 0, 16, packed, gs, bias=bias.to(DEV))
    What = oracle.dequant_grouped(pw["packed"], pw["scale"], GW)
    y64 = oracle.to_f64(X) @ What.T + oracle.to_f64(bias)[None, :]
    check_rows(y, y64, tag)
    # the oracle's own packed weights give the same bar
    y2 = w4.w4_linear_grouped(X.to(DEV), 0, 16, to_dev(pw["packed"]), to_dev(pw["scale"]), bias=bias.to(DEV))
    check_rows(y2, y64, tag + " (oracle weights)")


def test_attn_proj_w4a16():
    d = synth.attn_proj()
    w4a16_case(d["X"], d["W"], d["bias"], "attn_proj_w4a16")


@pytest.mark.parametrize("M,K", [(1, 4096), (16, 4096), (1, 12288), (16, 12288)])
def test_small_m_w4a16(M, K):
    N = 12288 if K == 4096 else 4096
    d = synth.small_m(M, K, N)
    w4a16_case(d["X"], d["W"], d["bias"], "small_m_w4a16 M=%d K=%d" % (M, K))
