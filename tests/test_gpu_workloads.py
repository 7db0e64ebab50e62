"""Full-size parity of the HIP path on the five DiT / text-encoder workloads (needs an MI355X).

Inputs come from ``synth`` (seeded, synthetic, the workloads' shapes and value
distributions).  Where the oracle cannot afford every output, it computes a seeded
sample of token rows (rows are independent: the per-token scale and the GEMM row
only depend on that row) and the GPU result is compared on those rows.  The GPU
always runs the full shape, in the same launch configuration as ``bench.py``.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import int4_weight_quantized_block_amd as w4
from parity import check_codes, check_scales, np_, rel_frob, sample_rows, FROB_TOL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def weights_on_gpu(W, g, asym):
    """Pack on the GPU and check the packing against the oracle; returns (gpu tensors, oracle dict)."""
    ref = oracle.pack_weights(W, g, asym)
    packed, s, zp = w4.w4_pack_weights(W.to(DEV), g, asym)
    Wr = ref["rotated"]
    unr = ((np.maximum(Wr.max(1), 0) - np.minimum(Wr.min(1), 0)) / 15.0) if asym else np.abs(Wr).max(1) / 7.0
    assert check_scales(np_(s), ref["scale"], unr, "row_scale").all()
    pg = np_(packed)
    if asym:
        assert np.array_equal(np_(zp), ref["zp"])
        check_codes(oracle.unpack_nibbles(pg, False), ref["codes"], ref["pre"] + ref["zp"][:, None], "w codes")
    else:
        check_codes(oracle.unpack_nibbles(pg, True), ref["codes"], ref["pre"], "w codes")
    return (packed, s, zp), ref


def check_layer(X, W, bias, g, bits, asym, rows, lowrank=None, cache=None, tag=""):
    """Run one linear on the GPU at full size and check it against the oracle.

    rows: token rows the oracle recomputes (None = all).  Returns (Y_gpu, oracle_y64 on rows)."""
    M, K = X.shape
    N = W.shape[0]
    say("%s: M=%d K=%d N=%d g=%d bits=%d asym=%s rows=%s" % (tag, M, K, N, g, bits, asym,
                                                           "all" if rows is None else len(rows)))
    (packed, s_w, zp), pw = weights_on_gpu(W, g, asym)
    Xd = X if X.is_cuda else X.to(DEV)
    Xc = X.cpu() if X.is_cuda else X
    if cache is not None:
        q, sx, rs = cache.get(Xd, g, bits)
    else:
        q, sx, rs = w4.w4_rotate_quant_act(Xd, g, bits)
    Xr = Xc if rows is None else Xc[torch.as_tensor(rows)]
    ra = oracle.rotate_quant_act(Xr, g, bits)
    sel = slice(None) if rows is None else rows
    sxg = np_(sx)[sel]
    amax64 = np.abs(ra["rotated"]).max(1) / oracle.QMAX[bits]
    assert check_scales(sxg, ra["scale"], amax64, tag + " tok_scale").all()
    qg = np_(q)[sel]
    codes = oracle.unpack_nibbles(qg, True) if bits == 4 else qg
    check_codes(codes, ra["q"], ra["pre"], tag + " act codes")
    # exact accumulators on the oracle's codes (all rows of the oracle's own quantized X)
    if rows is None:
        qo, so, rso = ra["q"], ra["scale"], ra["rowsum"]
    else:
        full = oracle.rotate_quant_act(Xc, g, bits)
        qo, so, rso = full["q"], full["scale"], full["rowsum"]
    qa = qo if bits == 8 else oracle.pack_nibbles(qo)
    acc_g = w4.w4_linear_cached_rot(to_dev(qa), to_dev(so), to_dev(rso.astype(np.int32)), bits,
                                    to_dev(pw["packed"]), to_dev(pw["scale"]),
                                    to_dev(pw["zp"]) if asym else None, out_i32=True)
    acc_o = oracle.gemm_i64(ra["q"], oracle.weight_operand(pw["packed"], pw["zp"], asym))
    assert np.array_equal(np_(acc_g)[sel].astype(np.int64), acc_o), tag + " accumulators"
    # the bf16 layer output (GPU rotation + GPU packing, as in the timed path)
    lr64 = None
    if lowrank is not None:
        L1, L2, low = lowrank
        lr64 = oracle.lowrank(Xr, L1.cpu().t(), L2.cpu())  # L1 is held rank-major, [r, K]
    y = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, bias=bias.to(DEV), lowrank=low if lowrank else None)
    y64 = oracle.epilogue(acc_o, ra["scale"], pw["scale"], bias.cpu(), lr64)
    err = rel_frob(y[torch.as_tensor(sel).to(DEV)] if rows is not None else y, y64)
    say("  %s rel frob %.3e" % (tag, err))
    assert err <= FROB_TOL, (tag, err)
    if cache is None:  # the uncached entry point gives the same bits
        y2 = w4.w4_linear(Xd, g, bits, packed, s_w, zp, bias=bias.to(DEV), lowrank=low if lowrank else None)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), tag + " w4_linear vs cached"
    return y, y64


def test_tiny_w4a8_g64():
    d = synth.tiny()
    check_layer(d["X"], d["W"], d["bias"], 64, 8, False, None, tag="tiny")


def test_attn_proj_w4a8_g256():
    d = synth.attn_proj()
    rows = sample_rows(d["X"].shape[0], 96, seed=1)
    check_layer(d["X"], d["W"], d["bias"], 256, 8, False, rows, tag="attn_proj")


def test_mlp_pair_w4a4_g256():
    up = synth.mlp_up()
    M = up["X"].shape[0]
    rows = sample_rows(M, 64, seed=2)
    check_layer(up["X"], up["W"], up["bias"], 256, 4, False, rows, tag="mlp_up")
    # host glue: GELU of the oracle's own up-projection output (all rows) feeds the down-proj
    say("oracle up-projection for the down-proj input (all %d rows)" % M)
    ref_up = oracle.linear(up["X"], up["W"], 256, 4, False, bias=up["bias"])
    h = oracle.gelu_bf16(ref_up["y"])
    dn = synth.mlp_down_weights()
    check_layer(h, dn["W"], dn["bias"], 256, 4, False, rows, tag="mlp_down")


@pytest.mark.parametrize("K,N", [(4096, 12288), (12288, 4096)])
@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_small_m_asym_w4a8(M, K, N):
    d = synth.small_m(M, K, N)
    check_layer(d["X"], d["W"], d["bias"], 256, 8, True, None, tag="small_m")


@pytest.mark.parametrize("b", [0, 19])
def test_double_block_cached_lowrank(b):
    """One DiT double block: QKV and MLP-up share the rotated block input through the cache;
    every linear carries a rank-32 low-rank branch on its unrotated input."""
    say("double block %d: drawing inputs on the GPU" % b)
    blk = synth.double_block(b, DEV)
    M = blk["x"].shape[0]
    rows = sample_rows(M, 48, seed=100 + b)
    cache = w4.RotationCache()
    outs = {}
    for name, inp in (("qkv", blk["x"]), ("up", blk["x"]), ("out", blk["attn"])):
        p = blk[name]
        t = w4.w4_lowrank_down(inp, p["L1"])
        low = w4.LowRank(l2=p["L2"], t=t)
        outs[name], _ = check_layer(inp, p["W"].cpu(), p["bias"], 256, 8, False, rows,
                                    lowrank=(p["L1"], p["L2"], low), cache=cache, tag="block%d.%s" % (b, name))
    assert cache.hits == 1 and cache.misses == 2
    # down-proj input: GELU of the oracle's up-projection output, all rows
    p = blk["up"]
    say("oracle up-projection + low-rank for the down-proj input (all %d rows)" % M)
    ref_up = oracle.linear(blk["x"].cpu(), p["W"].cpu(), 256, 8, False, bias=p["bias"].cpu(),
                           L1=p["L1"].cpu().t(), L2=p["L2"].cpu())
    h = oracle.gelu_bf16(ref_up["y"]).to(DEV)
    p = blk["down"]
    low = w4.LowRank(l2=p["L2"], x=h, l1=p["L1"])
    check_layer(h, p["W"].cpu(), p["bias"], 256, 8, False, rows, lowrank=(p["L1"], p["L2"], low),
                tag="block%d.down" % b)
    cache.clear()
