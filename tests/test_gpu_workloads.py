"""Full-size parity of the HIP path on the five DiT / text-encoder workloads (needs an MI355X).

Inputs come from ``synth`` (seeded, synthetic, the workloads' shapes and value
distributions).  The oracle computes every output: activation codes and scales of every
token, the int64 GEMM over all M x N accumulators, and the fp64 epilogue of every row
(the int64 loop takes tens of seconds per linear at these sizes).  The GPU runs the full
shape, in the same launch configuration as ``bench.py``.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import int4_weight_quantized_block_amd as w4
from parity import check_codes, check_scales, np_, rel_frob, FROB_TOL

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


def check_layer(X, W, bias, g, bits, asym, lowrank=None, cache=None, tag="", codes=None, keep=None):
    """Run one linear on the GPU at full size and check it against the oracle on every row.

    Checked: the GPU's packed weights and scales; its token scales and activation codes; the
    int32 accumulators of the oracle's own codes (exact, all M x N); the bf16 layer output of
    the GPU's own rotation and packing, as in the timed path (relative Frobenius error over
    all M x N).  Returns (Y_gpu, oracle y64); ``keep`` (a dict) receives the GPU's packed
    weights (packed, scales, zero points)."""
    M, K = X.shape
    N = W.shape[0]
    say("%s: M=%d K=%d N=%d g=%d bits=%d asym=%s" % (tag, M, K, N, g, bits, asym))
    (packed, s_w, zp), pw = weights_on_gpu(W, g, asym)
    if keep is not None:
        keep.update(packed=packed, s_w=s_w, zp=zp)
    Xd = X if X.is_cuda else X.to(DEV)
    Xc = X.cpu() if X.is_cuda else X
    if codes is not None:
        q, sx, rs = codes
    elif cache is not None:
        q, sx, rs = cache.get(Xd, g, bits)
    else:
        q, sx, rs = w4.w4_rotate_quant_act(Xd, g, bits)
    ra = oracle.rotate_quant_act(Xc, g, bits)
    amax64 = np.abs(ra["rotated"]).max(1) / oracle.QMAX[bits]
    assert check_scales(np_(sx), ra["scale"], amax64, tag + " tok_scale").all()
    qg = np_(q)
    codes = oracle.unpack_nibbles(qg, True) if bits == 4 else qg
    check_codes(codes, ra["q"], ra["pre"], tag + " act codes")
    # exact accumulators on the oracle's codes, every row
    qa = ra["q"] if bits == 8 else oracle.pack_nibbles(ra["q"])
    acc_g = w4.w4_linear_cached_rot(to_dev(qa), to_dev(ra["scale"]), to_dev(ra["rowsum"].astype(np.int32)), bits,
                                    to_dev(pw["packed"]), to_dev(pw["scale"]),
                                    to_dev(pw["zp"]) if asym else None, out_i32=True)
    say("  oracle int64 GEMM over all %d x %d outputs" % (M, N))
    acc_o = oracle.gemm_i64(ra["q"], oracle.weight_operand(pw["packed"], pw["zp"], asym))
    bad = np.argwhere(np_(acc_g).astype(np.int64) != acc_o)
    assert bad.size == 0, "%s accumulators: %d mismatches, first at %s" % (tag, len(bad), bad[:4].tolist())
    del acc_g
    # the bf16 layer output (GPU rotation + GPU packing, as in the timed path), every row
    lr64 = None
    if lowrank is not None:
        L1, L2, low = lowrank
        lr64 = oracle.lowrank(Xc, L1.cpu().t(), L2.cpu())  # L1 is held rank-major, [r, K]
    y = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, bias=bias.to(DEV), lowrank=low if lowrank else None)
    y64 = oracle.epilogue(acc_o, ra["scale"], pw["scale"], bias.cpu(), lr64)
    err = rel_frob(y, y64)
    # every 32-row block of every output tile on its own (a tile-local fault cannot hide in
    # the global norm)
    worst = 0.0
    for m0 in range(0, M, 32):
        worst = max(worst, rel_frob(y[m0:m0 + 32], y64[m0:m0 + 32]))
    say("  %s rel frob %.3e (worst 32-row block %.3e)" % (tag, err, worst))
    assert err <= FROB_TOL, (tag, err)
    assert worst <= 2 * FROB_TOL, (tag, worst)
    if cache is None and codes is None:  # the uncached entry point gives the same bits
        y2 = w4.w4_linear(Xd, g, bits, packed, s_w, zp, bias=bias.to(DEV), lowrank=low if lowrank else None)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), tag + " w4_linear vs cached"
    return y, y64


def test_tiny_w4a8_g64():
    d = synth.tiny()
    check_layer(d["X"], d["W"], d["bias"], 64, 8, False, tag="tiny")


def test_attn_proj_w4a8_g256():
    d = synth.attn_proj()
    check_layer(d["X"], d["W"], d["bias"], 256, 8, False, tag="attn_proj")


def test_mlp_pair_w4a4_g256():
    up = synth.mlp_up()
    _, y64 = check_layer(up["X"], up["W"], up["bias"], 256, 4, False, tag="mlp_up")
    # host glue: GELU of the oracle's own up-projection output (all rows) feeds the down-proj
    h = oracle.gelu_bf16(oracle.bf16_rne(y64))
    del y64
    dn = synth.mlp_down_weights()
    check_layer(h, dn["W"], dn["bias"], 256, 4, False, tag="mlp_down")


@pytest.mark.parametrize("K,N", [(4096, 12288), (12288, 4096)])
@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_small_m_asym_w4a8(M, K, N):
    d = synth.small_m(M, K, N)
    check_layer(d["X"], d["W"], d["bias"], 256, 8, True, tag="small_m")


@pytest.mark.parametrize("b", [0, 19])
def test_double_block_cached_lowrank(b):
    """One DiT double block: QKV and MLP-up share the rotated block input through the cache,
    and their stacked L1 factors give both low-rank inputs t in the same pass; every linear
    carries a rank-32 low-rank branch on its unrotated input."""
    say("double block %d: drawing inputs on the GPU" % b)
    blk = synth.double_block(b, DEV)
    cache = w4.RotationCache()
    l1_x = torch.cat([blk["qkv"]["L1"], blk["up"]["L1"]], dim=0)   # stacked [64, K]
    r = blk["qkv"]["L1"].shape[0]
    outs, kept = {}, {}
    for name, inp, l1, cols in (("qkv", blk["x"], l1_x, slice(0, r)), ("up", blk["x"], l1_x, slice(r, 2 * r)),
                                ("out", blk["attn"], blk["out"]["L1"], slice(0, r))):
        p = blk[name]
        q, sx, rs, t = cache.get(inp, 256, 8, l1=l1)
        low = w4.LowRank(l2=p["L2"], t=t[:, cols])
        kept[name] = {"low": low}
        outs[name], y64 = check_layer(inp, p["W"].cpu(), p["bias"], 256, 8, False, lowrank=(p["L1"], p["L2"], low),
                                      codes=(q, sx, rs), tag="block%d.%s" % (b, name), keep=kept[name])
        if name == "up":
            h = oracle.gelu_bf16(oracle.bf16_rne(y64)).to(DEV)   # the down-proj input, all rows
        del y64
    # the timed path's launch: QKV and MLP-up as one grid on the shared codes; each output
    # equals its own call above bit for bit
    q, sx, rs, t = cache.get(blk["x"], 256, 8, l1=l1_x)
    pair = [w4.LinearOut(packed=kept[n]["packed"], row_scale=kept[n]["s_w"], bias=blk[n]["bias"].to(DEV),
                         lowrank=kept[n]["low"]) for n in ("qkv", "up")]
    for n, y in zip(("qkv", "up"), w4.w4_linear_cached_rot_multi(q, sx, rs, 8, pair)):
        assert torch.equal(y.view(torch.int16), outs[n].view(torch.int16)), "block%d.%s: one launch vs own call" % (b, n)
    del pair, kept
    assert cache.hits == 2 and cache.misses == 2
    # down-proj input: GELU of the oracle's up-projection output (computed above, all rows);
    p = blk["down"]
    q, sx, rs, t = w4.w4_rotate_quant_act_lowrank(h, 256, 8, p["L1"])
    low = w4.LowRank(l2=p["L2"], t=t)
    check_layer(h, p["W"].cpu(), p["bias"], 256, 8, False, lowrank=(p["L1"], p["L2"], low), codes=(q, sx, rs),
                tag="block%d.down" % b)
    cache.clear()
