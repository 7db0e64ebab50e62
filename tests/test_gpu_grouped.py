"""Parity of the rotation sizes 16 / 1024 / 4096 and of the grouped-scale weight format
(per-(row, group) fp16 scales; W4A8, W4A4 and W4A16) against the CPU oracle (needs an MI355X).

Each test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle
import int4_weight_quantized_block_amd as w4
from parity import check_codes, check_scales, np_, rel_frob, FROB_TOL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def act_input(M, K, seed, dtype=torch.bfloat16, scale=30.0):
    r = rng(seed)
    x = r.standard_normal((M, K)).astype(np.float32)
    x[:, r.choice(K, max(1, K // 100), replace=False)] *= scale
    return torch.from_numpy(x).to(dtype)


def weights(N, K, seed, dtype=torch.bfloat16):
    r = rng(seed)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    # groups of very different magnitude, so a wrong group scale shows
    w *= np.exp(r.uniform(-2, 2, size=(N, K // 32))).repeat(32, axis=1).astype(np.float32)
    return torch.from_numpy(w).to(dtype)


def near_f16_midpoint(v: float, rel=2.0 ** -40) -> bool:
    s = np.float16(v)
    for nb in (np.nextafter(s, np.float16(np.inf)), np.nextafter(s, np.float16(-np.inf))):
        mid = (float(s) + float(nb)) / 2
        if abs(v - mid) <= rel * abs(v):
            return True
    return False


# --------------------------------------------------------------------------- rotation sizes
@pytest.mark.parametrize("M,K,g,bits,dtype", [
    (16, 256, 16, 8, torch.float32), (33, 3072, 16, 4, torch.bfloat16), (7, 3072, 1024, 8, torch.bfloat16),
    (300, 4096, 1024, 4, torch.bfloat16), (5, 12288, 4096, 8, torch.bfloat16), (64, 8192, 4096, 4, torch.float32),
    (1, 4096, 4096, 8, torch.bfloat16), (129, 1024, 16, 8, torch.bfloat16),
])
def test_rotate_quant_rotation_sizes(M, K, g, bits, dtype):
    say("rotquant g=%d M=%d K=%d bits=%d %s" % (g, M, K, bits, dtype))
    X = act_input(M, K, seed=M + K + g, dtype=dtype)
    X[M // 2] = 0
    ref = oracle.rotate_quant_act(X, g, bits)
    q, s, rs = w4.w4_rotate_quant_act(X.to(DEV), g, bits)
    amax64 = np.abs(ref["rotated"]).max(axis=1) / oracle.QMAX[bits]
    assert check_scales(np_(s), ref["scale"], amax64, "tok_scale").all()
    qg = np_(q)
    codes = oracle.unpack_nibbles(qg, signed=True) if bits == 4 else qg
    check_codes(codes, ref["q"], ref["pre"], "act codes")
    assert np.array_equal(np_(rs).astype(np.int64), codes.astype(np.int64).sum(1))
    assert np_(s)[M // 2] == 0 and np.all(codes[M // 2] == 0)


@pytest.mark.parametrize("N,K,g,asym", [(40, 256, 16, False), (33, 4096, 1024, True), (17, 12288, 4096, False),
                                        (64, 8192, 4096, True)])
def test_pack_rotation_sizes(N, K, g, asym):
    say("pack g=%d N=%d K=%d asym=%s" % (g, N, K, asym))
    W = weights(N, K, seed=N + K + g)
    ref = oracle.pack_weights(W, g, asym)
    packed, s, zp = w4.w4_pack_weights(W.to(DEV), g, asym)
    Wr = ref["rotated"]
    unr = (np.maximum(Wr.max(1), 0) - np.minimum(Wr.min(1), 0)) / 15.0 if asym else np.abs(Wr).max(1) / 7.0
    assert check_scales(np_(s), ref["scale"], unr, "row_scale").all()
    codes = oracle.unpack_nibbles(np_(packed), signed=not asym)
    if asym:
        assert np.array_equal(np_(zp), ref["zp"])
        check_codes(codes, ref["codes"], ref["pre"] + ref["zp"].astype(np.float64)[:, None], "w codes")
    else:
        check_codes(codes, ref["codes"], ref["pre"], "w codes")


@pytest.mark.parametrize("M,N,K,g,bits", [(300, 520, 3072, 1024, 8), (8, 1000, 4096, 4096, 4), (130, 96, 256, 16, 8)])
def test_linear_rotation_sizes(M, N, K, g, bits):
    say("linear g=%d M=%d N=%d K=%d bits=%d" % (g, M, N, K, bits))
    X = act_input(M, K, seed=3 * M + K)
    W = weights(N, K, seed=N + 7)
    bias = torch.from_numpy((rng(N).standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16)
    ref = oracle.linear(X, W, g, bits, False, bias=bias)
    packed, s_w, _ = w4.w4_pack_weights(W.to(DEV), g, False)
    y = w4.w4_linear(X.to(DEV), g, bits, packed, s_w, bias=bias.to(DEV))
    err = rel_frob(y, ref["y64"])
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL


# --------------------------------------------------------------------------- grouped pack
@pytest.mark.parametrize("N,K,g,gw,dtype", [
    (64, 256, 0, 32, torch.float32), (40, 3072, 256, 64, torch.bfloat16), (33, 4096, 0, 128, torch.bfloat16),
    (17, 12288, 1024, 256, torch.bfloat16), (8, 8192, 4096, 32, torch.float32), (50, 1024, 16, 64, torch.bfloat16),
])
def test_pack_grouped_matches_oracle(N, K, g, gw, dtype):
    say("pack grouped N=%d K=%d g=%d gw=%d %s" % (N, K, g, gw, dtype))
    W = weights(N, K, seed=N * 3 + K + gw, dtype=dtype)
    z = max(g, gw)
    W[1, :z] = 0                       # zero groups (whole rotation groups, so they stay zero)
    ref = oracle.pack_weights_grouped(W, g, gw)
    packed, gs = w4.w4_pack_weights_grouped(W.to(DEV), g, gw)
    assert gs.shape == (N, K // gw) and gs.dtype == torch.float16
    sg, so = np_(gs), ref["scale"]
    diff = sg.view(np.uint16) != so.view(np.uint16)
    if diff.any():   # only where fp64 max|w'|/7 sits on an fp16 rounding midpoint
        G = ref["rotated"].reshape(N, K // gw, gw)
        unr = np.abs(G).max(2) / 7.0
        for idx in np.argwhere(diff):
            assert near_f16_midpoint(float(unr[tuple(idx)])), idx
    assert np.all(sg[1, :z // gw] == 0.0)
    codes = oracle.unpack_nibbles(np_(packed), signed=True)
    rows_ok = ~diff.any(1)
    check_codes(codes[rows_ok], ref["codes"][rows_ok], ref["pre"][rows_ok], "grouped w codes")
    assert np.all(codes[1, :z] == 0)


# --------------------------------------------------------------------------- grouped layer
def grouped_case(M, N, K, g, gw, bits, seed, lr_rank=0, bias_dtype=torch.bfloat16):
    X = act_input(M, K, seed=seed)
    W = weights(N, K, seed=seed + 1)
    r = rng(seed + 2)
    bias = None
    if bias_dtype is not None:
        bias = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(bias_dtype)
    L1 = L2 = None
    if lr_rank:
        L1 = torch.from_numpy((r.standard_normal((K, lr_rank)) * 0.02).astype(np.float32)).to(torch.bfloat16)
        L2 = torch.from_numpy((r.standard_normal((lr_rank, N)) * 0.2).astype(np.float32)).to(torch.bfloat16)
    ref = oracle.linear_grouped(X, W, g, gw, bits, bias=bias, L1=L1, L2=L2)
    return X, W, bias, L1, L2, ref


@pytest.mark.parametrize("M,N,K,g,gw,bits,lr", [
    (300, 520, 3072, 256, 64, 8, False),      # large M, ragged tiles
    (257, 384, 4096, 256, 128, 4, True),      # W4A4, low-rank
    (130, 200, 1024, 64, 32, 8, False),       # gw = 32: two groups per stage
    (512, 256, 2048, 1024, 256, 8, True),
    (40, 1000, 4096, 256, 128, 8, False),     # 33..64 tokens
    (8, 4096, 12288, 256, 256, 8, True),      # few tokens, K split
    (1, 3000, 4096, 16, 64, 4, False),        # one token
    (20, 2048, 3072, 256, 32, 4, True),
    (16, 3000, 8192, 256, 64, 8, True),       # streaming form: 16 tokens, ragged N, low-rank
    (5, 1000, 3072, 64, 128, 4, False),       # streaming form, 4 waves (K not whole 2048-k stages)
    (2, 12288, 12288, 256, 128, 8, True),     # streaming form, N past 16 rows per CU
    (16, 16384, 4096, 256, 256, 4, False),    # streaming form, 64 rows per workgroup
])
def test_linear_grouped_int_matches_oracle(M, N, K, g, gw, bits, lr):
    """W4A8 / W4A4 with grouped fp16 weight scales: the raw integer sums on the oracle's codes
    are exact, the bf16 output is within the bar of the oracle's grouped fp64 epilogue."""
    say("grouped int M=%d N=%d K=%d g=%d gw=%d bits=%d lr=%s" % (M, N, K, g, gw, bits, lr))
    X, W, bias, L1, L2, ref = grouped_case(M, N, K, g, gw, bits, seed=M + N + K + gw, lr_rank=16 if lr else 0)
    pw = ref["w"]
    packed, gs = to_dev(pw["packed"]), to_dev(pw["scale"])
    qa = ref["a"]["q"] if bits == 8 else ref["a"]["packed"]
    acc = w4.w4_linear_cached_rot_grouped(to_dev(qa), to_dev(ref["a"]["scale"]), bits, packed, gs, out_i32=True)
    assert np.array_equal(np_(acc).astype(np.int64), ref["acc"])
    Xd = X.to(DEV)
    low = w4.LowRank(l2=L2.to(DEV), x=Xd, l1=L1.t().contiguous().to(DEV)) if lr else None
    # the GPU's own packing and rotation, as in the timed path
    packed_g, gs_g = w4.w4_pack_weights_grouped(W.to(DEV), g, gw)
    y = w4.w4_linear_grouped(Xd, g, bits, packed_g, gs_g, bias=bias.to(DEV), lowrank=low)
    err = rel_frob(y, ref["y64"])
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL
    # cached half with the oracle's codes and weights gives the same bar
    y2 = w4.w4_linear_cached_rot_grouped(to_dev(qa), to_dev(ref["a"]["scale"]), bits, packed, gs,
                                         bias=bias.to(DEV), lowrank=low)
    assert rel_frob(y2, ref["y64"]) <= FROB_TOL
    if lr:
        assert rel_frob(torch.from_numpy(ref["y64"] - ref["lr"]), ref["y64"]) > 4 * FROB_TOL


@pytest.mark.parametrize("M,N,K,gw,lr,bias_dtype", [
    (300, 520, 3072, 64, False, torch.bfloat16),
    (4096, 384, 1024, 128, True, torch.bfloat16),
    (257, 1000, 2048, 32, False, torch.float32),
    (64, 3072, 3072, 128, True, torch.bfloat16),
    (16, 4096, 4096, 256, False, None),
    (1, 12288, 4096, 128, False, torch.bfloat16),
    (33, 777, 12288, 64, True, torch.bfloat16),
    (3, 1000, 2048, 64, True, torch.float32),     # streaming form, gw = 64, low-rank
    (16, 12288, 3072, 64, False, torch.bfloat16),  # streaming form, 48 rows per workgroup
    (9, 520, 1024, 256, True, None),              # streaming form, one stage
])
def test_linear_w4a16_matches_oracle(M, N, K, gw, lr, bias_dtype):
    """W4A16 (no rotation): bf16 activations times the grouped int4 weights on the bf16 matrix
    cores, within the bar of the oracle's fp64 product with the dequantized weights."""
    say("w4a16 M=%d N=%d K=%d gw=%d lr=%s bias=%s" % (M, N, K, gw, lr, bias_dtype))
    X, W, bias, L1, L2, ref = grouped_case(M, N, K, 0, gw, 16, seed=M + 3 * N + K, lr_rank=16 if lr else 0,
                                           bias_dtype=bias_dtype)
    Xd = X.to(DEV)
    packed, gs = w4.w4_pack_weights_grouped(W.to(DEV), 0, gw)
    low = w4.LowRank(l2=L2.to(DEV), x=Xd, l1=L1.t().contiguous().to(DEV)) if lr else None
    y = w4.w4_linear_grouped(Xd, 0, 16, packed, gs, bias=bias.to(DEV) if bias is not None else None, lowrank=low)
    err = rel_frob(y, ref["y64"])
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL
    # the oracle's own packed weights give the same bar
    y2 = w4.w4_linear_grouped(Xd, 0, 16, to_dev(ref["w"]["packed"]), to_dev(ref["w"]["scale"]),
                              bias=bias.to(DEV) if bias is not None else None, lowrank=low)
    assert rel_frob(y2, ref["y64"]) <= FROB_TOL


def test_grouped_ksplit_equals_single_pass():
    """17 to 64 tokens with and without the workspace that splits K: integer sums identical,
    bf16 outputs within the bar of each other (the fp32 group sums are added in another order)."""
    M, N, K, gw = 24, 2048, 8192, 128
    say("grouped split M=%d N=%d K=%d gw=%d" % (M, N, K, gw))
    need = w4.w4_grouped_workspace_bytes(M, N, K, 8, gw)
    assert need > 0
    X, W, bias, _, _, ref = grouped_case(M, N, K, 256, gw, 8, seed=5)
    packed, gs = w4.w4_pack_weights_grouped(W.to(DEV), 256, gw)
    q, sx, _ = w4.w4_rotate_quant_act(X.to(DEV), 256, 8)
    big = torch.empty(need, dtype=torch.uint8, device=DEV)
    tiny = torch.empty(256, dtype=torch.uint8, device=DEV)
    a1 = w4.w4_linear_cached_rot_grouped(q, sx, 8, packed, gs, out_i32=True, ws=big)
    a0 = w4.w4_linear_cached_rot_grouped(q, sx, 8, packed, gs, out_i32=True, ws=tiny)
    assert torch.equal(a1, a0)
    y1 = w4.w4_linear_cached_rot_grouped(q, sx, 8, packed, gs, bias=bias.to(DEV), ws=big)
    y0 = w4.w4_linear_cached_rot_grouped(q, sx, 8, packed, gs, bias=bias.to(DEV), ws=tiny)
    assert rel_frob(y1, ref["y64"]) <= FROB_TOL and rel_frob(y0, ref["y64"]) <= FROB_TOL
    Xd = X.to(DEV)
    z1 = w4.w4_linear_grouped(Xd, 0, 16, packed, gs, ws=torch.empty(w4.w4_linear_grouped_workspace_bytes(M, N, K, 16, gw),
                                                                       dtype=torch.uint8, device=DEV))
    z0 = w4.w4_linear_grouped(Xd, 0, 16, packed, gs, ws=tiny)
    assert ((z1.float() - z0.float()).norm() / z0.float().norm()).item() <= 1e-3


def test_grouped_rejects_bad_arguments():
    X = torch.zeros((4, 256), dtype=torch.bfloat16, device=DEV)
    packed = torch.zeros((64, 128), dtype=torch.uint8, device=DEV)
    gs = torch.ones((64, 4), dtype=torch.float16, device=DEV)
    with pytest.raises(w4.W4Error) as e:
        w4.w4_linear_grouped(X, 64, 16, packed, gs)          # W4A16 with a rotation
    assert e.value.status == w4.W4_ERR_UNSUPPORTED
    with pytest.raises(w4.W4Error) as e:
        w4.w4_linear_grouped(X, 0, 8, packed, gs)            # integer activations need a rotation
    assert e.value.status == w4.W4_ERR_UNSUPPORTED
    with pytest.raises(w4.W4Error) as e:
        w4.w4_linear_grouped(X, 0, 16, packed, gs, out_i32=True)
    assert e.value.status == w4.W4_ERR_INVALID_ARG
    with pytest.raises(w4.W4Error) as e:
        w4.w4_pack_weights_grouped(torch.zeros((8, 256), device=DEV), 64, 16)
    assert e.value.status == w4.W4_ERR_UNSUPPORTED
