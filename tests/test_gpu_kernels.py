"""Kernel-level parity of the HIP path against the CPU oracle (needs an MI355X).

Each test prints what it runs before touching the GPU, so a failing case is named
even if the process dies.
"""
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


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def act_input(M, K, seed, dtype=torch.bfloat16, n_out=None, scale=30.0):
    r = rng(seed)
    x = r.standard_normal((M, K)).astype(np.float32)
    n_out = max(1, K // 100) if n_out is None else n_out
    x[:, r.choice(K, n_out, replace=False)] *= scale
    return torch.from_numpy(x).to(dtype)


# --------------------------------------------------------------------------- integer GEMM
@pytest.mark.parametrize("M,N,K,bits,asym", [
    (16, 128, 256, 8, False), (1, 64, 256, 8, True), (5, 48, 320, 8, False), (64, 256, 512, 4, False),
    (33, 272, 1024, 4, True), (128, 128, 256, 8, False), (200, 136, 448, 8, True), (300, 520, 3072, 4, False),
    (257, 256, 4096, 8, False), (130, 1000, 192, 4, True), (65, 17, 64, 8, False),
    (70, 64, 32768, 8, True), (8, 96, 32768, 4, False),   # K = W4_MAX_K, both paths
    # small-M streaming launch shapes: 8 waves with whole 2048-k stages and with a K tail inside
    # a stage, 4 waves once the grid passes one workgroup per CU, 16 tokens over 3 and 4 row
    # blocks; ragged N throughout
    (3, 1000, 4096, 4, False), (7, 520, 3072, 8, True), (1, 4100, 2048, 8, True),
    (16, 9000, 2048, 4, True), (12, 12300, 1024, 8, False),
])
def test_accumulators_bit_exact_on_oracle_codes(M, N, K, bits, asym):
    """acc[m, n] = sum_k q (c - z) from the oracle's own codes, through W4_OUT_I32."""
    say("acc exact M=%d N=%d K=%d bits=%d asym=%s" % (M, N, K, bits, asym))
    r = rng(M * 7 + N * 3 + K + bits + asym)
    qmax = oracle.QMAX[bits]
    q = r.integers(-qmax - 1, qmax + 1, size=(M, K)).astype(np.int8)
    if asym:
        codes = r.integers(0, 16, size=(N, K))
        zp = r.integers(0, 16, size=N).astype(np.uint8)
    else:
        codes = r.integers(-8, 8, size=(N, K))
        zp = None
    packed = oracle.pack_nibbles(codes)
    acc = oracle.gemm_i64(q, oracle.weight_operand(packed, zp, asym))
    qa = q if bits == 8 else oracle.pack_nibbles(q)
    y = w4.w4_linear_cached_rot(
        to_dev(qa), to_dev(np.ones(M, np.float32)), to_dev(q.astype(np.int64).sum(1).astype(np.int32)), bits,
        to_dev(packed), to_dev(np.ones(N, np.float32)), to_dev(zp) if asym else None, out_i32=True)
    got = np_(y).astype(np.int64)
    bad = np.argwhere(got != acc)
    assert bad.size == 0, "first mismatches %s: gpu %s oracle %s" % (
        bad[:4].tolist(), got[tuple(bad[:4].T)].tolist(), acc[tuple(bad[:4].T)].tolist())


@pytest.mark.parametrize("bits", [8, 4])
def test_accumulators_extreme_asym_max_k(bits):
    """The largest accumulators the kernels form: asymmetric weights (codes 15, zero point 0)
    against the most negative activation code at K = W4_MAX_K.  The kernels scale the
    operands by 16 (int8) or 256 (int4) and add (8 - z) * rowsum separately, so their int32
    intermediates reach about 1.0e9; the result must still be exact (GEMM and small-M)."""
    say("acc extreme asym bits=%d" % bits)
    N, K = 64, 32768
    qmin = -128 if bits == 8 else -8
    for M in (80, 8):
        q = np.full((M, K), qmin, np.int8)
        q[1::2] = 127 if bits == 8 else 7
        codes = np.full((N, K), 15)
        codes[1::2] = 0
        zp = np.zeros(N, np.uint8)
        zp[1::2] = 15
        packed = oracle.pack_nibbles(codes)
        acc = oracle.gemm_i64(q, oracle.weight_operand(packed, zp, True))
        qa = q if bits == 8 else oracle.pack_nibbles(q)
        y = w4.w4_linear_cached_rot(to_dev(qa), to_dev(np.ones(M, np.float32)),
                                    to_dev(q.astype(np.int64).sum(1).astype(np.int32)), bits, to_dev(packed),
                                    to_dev(np.ones(N, np.float32)), to_dev(zp), out_i32=True)
        assert np.array_equal(np_(y).astype(np.int64), acc)


def test_accumulators_extreme_codes():
    """All activation codes -128 against weight codes -8 (and 127 against 7) at K = 4096."""
    say("acc extremes")
    M, N, K = 80, 64, 4096
    q = np.full((M, K), -128, np.int8)
    q[1::2] = 127
    codes = np.full((N, K), -8)
    codes[1::2] = 7
    packed = oracle.pack_nibbles(codes)
    acc = oracle.gemm_i64(q, oracle.weight_operand(packed, None, False))
    for m in (M, 16):
        y = w4.w4_linear_cached_rot(to_dev(q[:m]), to_dev(np.ones(m, np.float32)),
                                    to_dev(q[:m].astype(np.int64).sum(1).astype(np.int32)), 8,
                                    to_dev(packed), to_dev(np.ones(N, np.float32)), out_i32=True)
        assert np.array_equal(np_(y).astype(np.int64), acc[:m])


# --------------------------------------------------------------------------- activations
@pytest.mark.parametrize("M,K,g,bits,dtype", [
    (16, 256, 64, 8, torch.float32), (16, 256, 256, 8, torch.bfloat16), (7, 3072, 256, 8, torch.bfloat16),
    (33, 3072, 256, 4, torch.bfloat16), (5, 12288, 256, 8, torch.bfloat16), (9, 12288, 256, 4, torch.bfloat16),
    (3, 4096, 256, 8, torch.bfloat16), (300, 768, 256, 8, torch.bfloat16), (21, 192, 64, 4, torch.float32),
    (40, 1280, 64, 8, torch.bfloat16), (2, 4608, 256, 8, torch.float32), (1, 64, 64, 4, torch.bfloat16),
    (37, 9472, 256, 8, torch.bfloat16), (3, 32768, 256, 4, torch.bfloat16), (1000, 256, 64, 8, torch.bfloat16),
    (129, 1024, 256, 4, torch.float32), (64, 2048, 64, 8, torch.bfloat16), (50, 6144, 256, 4, torch.bfloat16),
    (31, 3072, 64, 8, torch.bfloat16), (2100, 1024, 256, 8, torch.bfloat16), (600, 12288, 256, 8, torch.bfloat16),
])
def test_rotate_quant_act_matches_oracle(M, K, g, bits, dtype):
    say("rotquant M=%d K=%d g=%d bits=%d %s" % (M, K, g, bits, dtype))
    X = act_input(M, K, seed=M + K + g + bits, dtype=dtype)
    X[M // 2] = 0  # an all-zero token
    ref = oracle.rotate_quant_act(X, g, bits)
    q, s, rs = w4.w4_rotate_quant_act(X.to(DEV), g, bits)
    amax64 = np.abs(ref["rotated"]).max(axis=1) / oracle.QMAX[bits]
    eq = check_scales(np_(s), ref["scale"], amax64, "tok_scale")
    assert eq.all()
    qg = np_(q)
    if bits == 4:
        assert qg.shape == (M, K // 2)
        codes = oracle.unpack_nibbles(qg, signed=True)
    else:
        codes = qg
    n = check_codes(codes, ref["q"], ref["pre"], "act codes")
    if n == 0:
        want = ref["packed"] if bits == 4 else ref["q"].view(np.uint8)
        assert np.array_equal(qg.view(np.uint8), want)
    assert np.array_equal(np_(rs).astype(np.int64), codes.astype(np.int64).sum(1))
    assert np_(s)[M // 2] == 0 and np.all(codes[M // 2] == 0)


def test_rotate_quant_rejects_unsupported_k():
    # g = 64, K = 64 * 131: not a multiple of 256 (no streaming kernel), and K/16 = 524 chunks
    # have no split C * T with C <= 4, T % 4 == 0, T <= 512
    X = torch.zeros((2, 64 * 131), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w4.W4Error) as e:
        w4.w4_rotate_quant_act(X, 64, 8)
    assert e.value.status == w4.W4_ERR_UNSUPPORTED


# --------------------------------------------------------------------------- weights
@pytest.mark.parametrize("N,K,g,asym,dtype", [
    (256, 256, 64, False, torch.float32), (64, 3072, 256, False, torch.bfloat16),
    (48, 4096, 256, True, torch.bfloat16), (33, 12288, 256, True, torch.bfloat16),
    (17, 192, 64, True, torch.float32), (8, 9216, 256, False, torch.bfloat16),
])
def test_pack_weights_matches_oracle(N, K, g, asym, dtype):
    say("pack N=%d K=%d g=%d asym=%s %s" % (N, K, g, asym, dtype))
    r = rng(N + K)
    W = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(dtype)
    W[1] = 0  # zero row
    if N > 4:
        W[2] = W[2].abs() + 0.01  # all-positive row (asym: z = 0)
        W[3] = -(W[3].abs() + 0.01)
    ref = oracle.pack_weights(W, g, asym)
    packed, s, zp = w4.w4_pack_weights(W.to(DEV), g, asym)
    Wr = ref["rotated"]
    if asym:
        unr = (np.maximum(Wr.max(1), 0) - np.minimum(Wr.min(1), 0)) / 15.0
    else:
        unr = np.abs(Wr).max(1) / 7.0
    assert check_scales(np_(s), ref["scale"], unr, "row_scale").all()
    pg = np_(packed)
    assert pg.shape == (N, K // 2)
    codes = oracle.unpack_nibbles(pg, signed=not asym)
    if asym:
        zg = np_(zp)
        zdiff = zg != ref["zp"]
        if zdiff.any():  # only at a tie of -lo/s
            f = np.abs(ref["zpre"][zdiff] - np.floor(ref["zpre"][zdiff]) - 0.5)
            assert np.all(f <= 1e-6)
        pre = ref["pre"] + ref["zp"].astype(np.float64)[:, None]
        check_codes(codes[~zdiff], ref["codes"][~zdiff], pre[~zdiff], "weight codes")
    else:
        check_codes(codes, ref["codes"], ref["pre"], "weight codes")


# --------------------------------------------------------------------------- whole layer
@pytest.mark.parametrize("M,N,K,g,bits,asym,lr,bias_dtype", [
    (16, 256, 256, 64, 8, False, False, torch.bfloat16), (100, 200, 512, 256, 8, False, True, torch.bfloat16),
    (40, 96, 768, 256, 4, True, True, torch.bfloat16), (130, 64, 256, 64, 4, False, False, torch.bfloat16),
    (1, 300, 1024, 256, 8, True, False, torch.bfloat16), (97, 33, 320, 64, 8, True, False, torch.float32),
    (300, 401, 1024, 256, 4, False, False, torch.bfloat16), (77, 195, 256, 256, 8, False, False, None),
    (513, 389, 448, 64, 8, True, False, torch.float32),
])
def test_linear_matches_oracle(M, N, K, g, bits, asym, lr, bias_dtype):
    say("linear M=%d N=%d K=%d g=%d bits=%d asym=%s lr=%s bias=%s" % (M, N, K, g, bits, asym, lr, bias_dtype))
    r = rng(M + N + K)
    X = act_input(M, K, seed=M * 3 + K)
    W = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32))
    bias = bias.to(bias_dtype) if bias_dtype is not None else None
    L1 = L2 = None
    if lr:
        L1 = torch.from_numpy((r.standard_normal((K, 16)) * 0.01).astype(np.float32)).to(torch.bfloat16)
        L2 = torch.from_numpy((r.standard_normal((16, N)) * 0.01).astype(np.float32)).to(torch.bfloat16)
    ref = oracle.linear(X, W, g, bits, asym, bias=bias, L1=L1, L2=L2)
    pw = ref["w"]
    Xd = X.to(DEV)
    args = (to_dev(pw["packed"]), to_dev(pw["scale"]), to_dev(pw["zp"]) if asym else None)
    low = w4.LowRank(l2=L2.to(DEV), x=Xd, l1=L1.t().contiguous().to(DEV)) if lr else None
    bias_d = bias.to(DEV) if bias is not None else None
    y = w4.w4_linear(Xd, g, bits, *args, bias=bias_d, lowrank=low)
    err = rel_frob(y, ref["y64"])
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL
    # the same through the cached half, with a precomputed low-rank t
    q, s, rs = w4.w4_rotate_quant_act(Xd, g, bits)
    if lr:
        t = w4.w4_lowrank_down(Xd, L1.t().contiguous().to(DEV))
        tref = oracle.to_f64(X) @ oracle.to_f64(L1)
        assert np.abs(np_(t) - tref).max() <= 1e-4 * np.abs(tref).max()
        low = w4.LowRank(l2=L2.to(DEV), t=t)
    y2 = w4.w4_linear_cached_rot(q, s, rs, bits, *args, bias=bias_d, lowrank=low)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("M,N,K,bits,asym,r,tcol", [
    (300, 384, 512, 8, False, 32, None), (300, 389, 512, 8, True, 5, None), (260, 200, 768, 4, False, 20, None),
    (300, 392, 256, 4, True, 40, None), (257, 384, 512, 8, False, 64, None), (513, 191, 320, 8, False, 63, None),
    (8, 389, 512, 8, False, 20, None), (40, 384, 512, 4, True, 64, None),
    # large-M kernel with t and l2 staged in LDS (N % 8 == 0, r % 4 == 0, r <= 32): one,
    # two (K tail) and three stages, int4 codes with t past the ring, ragged M over three
    # tile rows, and t as a 16-byte aligned column range of a wider tensor
    (270, 256, 128, 8, True, 16, None), (300, 392, 192, 4, True, 12, None), (300, 384, 384, 8, True, 24, None),
    (100, 256, 64, 8, False, 16, None),
    (300, 200, 320, 4, False, 32, None), (520, 384, 1024, 8, False, 28, None), (300, 384, 512, 8, False, 32, 8),
    (300, 200, 512, 4, True, 16, 4),
    # t starting at float 2 (8-byte aligned): refused with W4_ERR_ALIGN before any launch
    (300, 384, 512, 8, False, 32, 2),
])
def test_linear_lowrank_ranks(M, N, K, bits, asym, r, tcol):
    """The low-rank branch at ranks that fill 1..4 k-steps of 16 (r % 4 != 0 included), with
    factors large enough that the branch carries a good part of the output; ragged N takes
    the element-wise l2 staging of the large-M kernel.  With tcol, t is columns tcol ..
    tcol + r of a wider f32 tensor (row stride r + 12)."""
    say("linear lowrank M=%d N=%d K=%d bits=%d asym=%s r=%d tcol=%s" % (M, N, K, bits, asym, r, tcol))
    g = 64
    rg = rng(7 * M + N + r)
    X = act_input(M, K, seed=M + 5 * r)
    W = torch.from_numpy((rg.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    L1 = torch.from_numpy((rg.standard_normal((K, r)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    L2 = torch.from_numpy((rg.standard_normal((r, N)) * 0.2).astype(np.float32)).to(torch.bfloat16)
    ref = oracle.linear(X, W, g, bits, asym, L1=L1, L2=L2)
    # the case can see a wrong branch: without it the output is far off
    assert rel_frob(torch.from_numpy(ref["y64"] - ref["lr"]), ref["y64"]) > 20 * FROB_TOL
    pw = ref["w"]
    Xd = X.to(DEV)
    args = (to_dev(pw["packed"]), to_dev(pw["scale"]), to_dev(pw["zp"]) if asym else None)
    t = w4.w4_lowrank_down(Xd, L1.t().contiguous().to(DEV))
    tref = oracle.to_f64(X) @ oracle.to_f64(L1)
    assert np.abs(np_(t) - tref).max() <= 1e-4 * np.abs(tref).max()
    if tcol is not None:
        wide = torch.full((M, r + 12), float("nan"), dtype=torch.float32, device=DEV)
        wide[:, tcol:tcol + r] = t
        t = wide[:, tcol:tcol + r]
        if tcol % 4:
            with pytest.raises(w4.W4Error, match="W4_ERR_ALIGN"):
                w4.w4_linear(Xd, g, bits, *args, lowrank=w4.LowRank(l2=L2.to(DEV), t=t))
            return
    y = w4.w4_linear(Xd, g, bits, *args, lowrank=w4.LowRank(l2=L2.to(DEV), t=t))
    err = rel_frob(y, ref["y64"])
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL


@pytest.mark.parametrize("M,K,Ns,bits,asym,ranks,i32", [
    (600, 1024, (960, 1280), 8, False, (32, 32), False),        # one launch, staged low-rank branches
    (300, 448, (389, 200, 384), 4, True, (28, 30, 0), False),   # K tail, generic low-rank, ragged N; third alone
    (520, 512, (384, 392), 8, True, (0, 0), True),              # raw accumulators
    (300, 512, (384, 256, 512), 8, False, (16, 0, 0), False),   # forms differ: 0 alone, 1 + 2 together
    (48, 1024, (512, 768), 8, False, (16, 16), False),          # M <= 64: the small-M kernels one by one
])
def test_linear_multi_equals_separate(M, K, Ns, bits, asym, ranks, i32):
    """Several linears on one set of codes: each output equals w4_linear_cached_rot's for the
    same linear bit for bit (large M, no split tail at these sizes), whether it shares a
    launch or not; the first case is also checked against the oracle.  The low-rank t of all
    outputs comes from one rotate-quant pass with the L1 factors stacked."""
    say("multi M=%d K=%d Ns=%s bits=%d asym=%s ranks=%s i32=%s" % (M, K, Ns, bits, asym, ranks, i32))
    g = 256 if K % 256 == 0 else 64
    rg = rng(M + K + sum(Ns))
    X = act_input(M, K, seed=M + 11 * K)
    Xd = X.to(DEV)
    Ws, L1s, L2s, biases = [], [], [], []
    for N, r in zip(Ns, ranks):
        Ws.append(torch.from_numpy((rg.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16))
        biases.append(torch.from_numpy((rg.standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16))
        L1s.append(torch.from_numpy((rg.standard_normal((K, r)) * 0.05).astype(np.float32)).to(torch.bfloat16)
                   if r else None)
        L2s.append(torch.from_numpy((rg.standard_normal((r, N)) * 0.2).astype(np.float32)).to(torch.bfloat16)
                   if r else None)
    stacked = [L1 for L1 in L1s if L1 is not None]
    if stacked:
        l1 = torch.cat([L1.t() for L1 in stacked], 0).contiguous().to(DEV)
        q, sx, rs, t = w4.w4_rotate_quant_act_lowrank(Xd, g, bits, l1)
    else:
        q, sx, rs = w4.w4_rotate_quant_act(Xd, g, bits)
    outs, lows, col = [], [], 0
    for W, b, r, L2 in zip(Ws, biases, ranks, L2s):
        packed, sw, zp = w4.w4_pack_weights(W.to(DEV), g, asym)
        low = w4.LowRank(l2=L2.to(DEV), t=t[:, col:col + r]) if r else None
        col += r
        lows.append(low)
        outs.append(w4.LinearOut(packed=packed, row_scale=sw, zp=zp, bias=b.to(DEV), lowrank=low, out_i32=i32))
    ys = w4.w4_linear_cached_rot_multi(q, sx, rs, bits, outs)
    tiny = torch.empty(256, dtype=torch.uint8, device=DEV) if M > 64 else None
    for i, (o, y) in enumerate(zip(outs, ys)):
        y1 = w4.w4_linear_cached_rot(q, sx, rs, bits, o.packed, o.row_scale, o.zp, bias=o.bias,
                                     lowrank=o.lowrank, out_i32=i32, ws=tiny)
        view = (lambda a: a) if i32 else (lambda a: a.view(torch.int16))
        assert torch.equal(view(y), view(y1)), "output %d differs from its own call" % i
    if ranks == (32, 32):
        for i, (W, b, L1, L2) in enumerate(zip(Ws, biases, L1s, L2s)):
            ref = oracle.linear(X, W, g, bits, asym, bias=b, L1=L1, L2=L2)
            err = rel_frob(ys[i], ref["y64"])
            say("  output %d rel frob %.3e" % (i, err))
            assert err <= FROB_TOL


@pytest.mark.parametrize("M,N,K,bits,asym", [(4608, 3072, 3072, 4, True), (4608, 2880, 2048, 8, False),
                                             (2500, 5996, 1024, 8, True)])
def test_gemm_split_tail_equals_single_pass(M, N, K, bits, asym):
    """More tiles than compute units: the last partial round runs as K ranges plus a sum and
    epilogue kernel (given the workspace).  The int32 outputs equal the single-pass kernel's
    bit for bit, the bf16 outputs too without a low-rank branch (same epilogue arithmetic) and
    within the bar with one (VALU instead of MFMA for T . L2)."""
    say("split tail M=%d N=%d K=%d bits=%d asym=%s" % (M, N, K, bits, asym))
    g = torch.Generator(device=DEV).manual_seed(M + N + K)
    X = torch.randn(M, K, generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn(N, K, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    bias = (torch.randn(N, generator=g, device=DEV) * 0.01).to(torch.bfloat16)
    L1t = (torch.randn(16, K, generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    L2 = (torch.randn(16, N, generator=g, device=DEV) * 0.2).to(torch.bfloat16)
    packed, s_w, zp = w4.w4_pack_weights(W, 256, asym)
    q, sx, rs = w4.w4_rotate_quant_act(X, 256, bits)
    L = w4.load_library()
    need = L.w4_workspace_bytes(M, N, K, bits, 0)
    assert need > 0, "shape must have a split tail"
    tiny = torch.empty(256, dtype=torch.uint8, device=DEV)   # too small: single pass
    big = torch.empty(need, dtype=torch.uint8, device=DEV)
    a1 = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, out_i32=True, ws=big)
    a0 = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, out_i32=True, ws=tiny)
    assert torch.equal(a1, a0)
    y1 = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, bias=bias, ws=big)
    y0 = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, bias=bias, ws=tiny)
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
    t = w4.w4_lowrank_down(X, L1t)
    low = w4.LowRank(l2=L2, t=t)
    y1 = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, bias=bias, lowrank=low, ws=big)
    y0 = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, zp, bias=bias, lowrank=low, ws=tiny)
    err = (y1.float() - y0.float()).norm() / y0.float().norm()
    say("  low-rank split vs single pass rel frob %.3e" % err.item())
    assert err.item() <= FROB_TOL


# --------------------------------------------------------------------------- fused small-M path
@pytest.mark.parametrize("M,N,K,g,bits,asym,bias_dtype,lr", [
    (1, 4096, 12288, 256, 8, True, torch.bfloat16, False),   # text-encoder shape, fused
    (1, 1000, 8192, 64, 4, True, None, False),               # fused W4A4, g = 64, ragged N
    (1, 520, 4096, 256, 4, False, torch.bfloat16, True),     # fused W4A4, low-rank, ragged N
    (1, 300, 16384, 64, 8, False, None, False),              # fused, largest K (8 stages, ring of 2)
    (1, 64, 2048, 256, 8, True, torch.float32, True),        # fused, one stage (fewer than the ring)
    (1, 8192, 4096, 256, 8, True, torch.bfloat16, False),    # fused, 32 rows per workgroup
    (1, 4100, 4096, 256, 8, True, torch.bfloat16, False),    # fused, 32 rows per workgroup, ragged N
    (1, 700, 3072, 256, 8, True, torch.bfloat16, True),      # fused with 12 waves, one stage, low-rank
    (1, 2000, 6144, 64, 4, False, None, False),              # fused with 12 waves, 2 stages = the ring
    (1, 12288, 4096, 256, 8, True, torch.bfloat16, False),   # past 32 rows per CU: two launches
    (1, 12300, 2048, 64, 4, True, torch.bfloat16, True),     # two launches, ragged N
    (2, 2048, 4096, 256, 8, True, torch.bfloat16, True),     # two tokens: two launches
    (4, 1000, 4096, 256, 8, False, torch.float32, True),     # two launches
])
def test_fused_small_m_equals_two_launches(M, N, K, g, bits, asym, bias_dtype, lr):
    """w4_linear at one token rotates, quantizes and multiplies in one launch; its output must
    equal w4_rotate_quant_act followed by w4_linear_cached_rot bit for bit, for bf16 and raw
    int32 outputs (the rotate-quant kernel itself is pinned to the oracle elsewhere).  The
    cases next to the fusion limits check the same equality on the two-launch side."""
    say("fused small-M M=%d N=%d K=%d g=%d bits=%d asym=%s bias=%s lr=%s" % (M, N, K, g, bits, asym, bias_dtype, lr))
    r = rng(M * 11 + N + K + g + bits)
    X = act_input(M, K, seed=M + 3 * K).to(DEV)
    W = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16).to(DEV)
    packed, scale, zp = w4.w4_pack_weights(W, g, asym)
    bias = None
    if bias_dtype is not None:
        bias = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(bias_dtype).to(DEV)
    low = None
    if lr:
        L1t = torch.from_numpy((r.standard_normal((16, K)) * 0.01).astype(np.float32)).to(torch.bfloat16).to(DEV)
        L2 = torch.from_numpy((r.standard_normal((16, N)) * 0.05).astype(np.float32)).to(torch.bfloat16).to(DEV)
        low = w4.LowRank(l2=L2, x=X, l1=L1t)
    y1 = w4.w4_linear(X, g, bits, packed, scale, zp, bias=bias, lowrank=low)
    q, s, rs = w4.w4_rotate_quant_act(X, g, bits)
    y2 = w4.w4_linear_cached_rot(q, s, rs, bits, packed, scale, zp, bias=bias, lowrank=low)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    a1 = w4.w4_linear(X, g, bits, packed, scale, zp, out_i32=True)
    a2 = w4.w4_linear_cached_rot(q, s, rs, bits, packed, scale, zp, out_i32=True)
    assert torch.equal(a1, a2)
    assert bool(torch.isfinite(y1.float()).all()) and float(y1.float().abs().max()) > 0


@pytest.mark.parametrize("asym", [False, True])
def test_fused_small_m_zero_token(asym):
    """An all-zero token through the fused launch: token scale 0, codes 0, so the output is the
    bias alone (rounded to bf16), and it equals the two-launch path bit for bit."""
    N, K = 2048, 4096
    say("fused small-M zero token N=%d K=%d asym=%s" % (N, K, asym))
    assert w4.w4_linear_fused(1, N, K, 256, 8)
    r = rng(N + K + asym)
    X = torch.zeros((1, K), dtype=torch.bfloat16, device=DEV)
    W = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16).to(DEV)
    bias = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16).to(DEV)
    packed, scale, zp = w4.w4_pack_weights(W, 256, asym)
    y1 = w4.w4_linear(X, 256, 8, packed, scale, zp, bias=bias)
    q, s, rs = w4.w4_rotate_quant_act(X, 256, 8)
    assert float(s[0]) == 0.0 and int(rs[0]) == 0 and not bool(q.any())
    y2 = w4.w4_linear_cached_rot(q, s, rs, 8, packed, scale, zp, bias=bias)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1[0].view(torch.int16), bias.view(torch.int16))


@pytest.mark.parametrize("M,N,K,g,bits,asym", [
    (1, 12300, 2048, 64, 4, True),     # 4 waves, 3 workgroups per CU, 2 stages = the ring depth
    (4, 12288, 1024, 256, 8, True),    # one stage
    (16, 8192, 2048, 256, 4, False),   # 16 tokens, 2 row blocks, 2 stages
    (8, 5000, 2048, 256, 8, True),     # ragged N
    (1, 2048, 2048, 256, 8, True),     # fused, one stage
    (1, 4096, 4096, 64, 8, True),      # fused, 2 stages = the ring depth
    (1, 3000, 3072, 256, 8, True),     # fused with 12 waves, one stage
])
def test_small_m_short_k_constants(M, N, K, g, bits, asym):
    """Small-M kernels whose whole K fits in the stages issued up front: the per-row constants
    (row scales, bias, zero points) must have landed before the epilogue reads them.  The
    bf16 output is the same on every launch, equals w4_linear's, and matches the fp64
    epilogue of the (exact) int32 accumulators."""
    say("small-M short K M=%d N=%d K=%d g=%d bits=%d asym=%s" % (M, N, K, g, bits, asym))
    r = rng(M + N + K + g + 3 * bits)
    X = act_input(M, K, seed=N + K).to(DEV)
    W = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16).to(DEV)
    bias = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16).to(DEV)
    packed, scale, zp = w4.w4_pack_weights(W, g, asym)
    q, s, rs = w4.w4_rotate_quant_act(X, g, bits)
    ys = [w4.w4_linear_cached_rot(q, s, rs, bits, packed, scale, zp, bias=bias) for _ in range(6)]
    yl = [w4.w4_linear(X, g, bits, packed, scale, zp, bias=bias) for _ in range(6)]
    for y in ys[1:] + yl:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    acc = np_(w4.w4_linear_cached_rot(q, s, rs, bits, packed, scale, zp, out_i32=True)).astype(np.int64)
    y64 = oracle.epilogue(acc, np_(s), np_(scale), bias.cpu())
    err = rel_frob(ys[0], y64)
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL


# --------------------------------------------------------------------------- K-split small-M path
@pytest.mark.parametrize("M,N,K,g,bits,asym", [
    (20, 4096, 12288, 256, 8, True),    # S = 8, text-encoder shape
    (24, 2000, 12288, 256, 8, False),   # S = 8, ragged N
    (40, 3072, 3072, 256, 4, False),    # S = 2, W4A4
    (33, 1000, 4096, 64, 4, True),      # S = 2, ragged N and M, W4A4 asymmetric
    (48, 1536, 3072, 256, 4, True),     # S = 2, three 16-token blocks
])
@pytest.mark.parametrize("lr_mode", ["none", "x", "t"])
def test_small_m_ksplit_matches_oracle(M, N, K, g, bits, asym, lr_mode):
    """17..48 tokens with a workspace: K is split over S > 1 workgroups whose int32 partial
    tiles k_gemv_reduce sums in a fixed order before the epilogue (asymmetric correction,
    low-rank term, bias).  Accumulators on the oracle's codes are exact; the layer output is
    within the bar of the oracle's fp64 output, with the branch given as (x, L1) or as t."""
    say("ksplit M=%d N=%d K=%d g=%d bits=%d asym=%s lr=%s" % (M, N, K, g, bits, asym, lr_mode))
    S = w4.w4_workspace_bytes(M, N, K, bits, 0) // (M * N * 4)
    assert S > 1, "shape must take the K-split path"
    r = rng(M * 13 + N + K + bits)
    X = act_input(M, K, seed=M + 7 * K)
    W = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16)
    L1 = torch.from_numpy((r.standard_normal((K, 16)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    L2 = torch.from_numpy((r.standard_normal((16, N)) * 0.2).astype(np.float32)).to(torch.bfloat16)
    lr = lr_mode != "none"
    ref = oracle.linear(X, W, g, bits, asym, bias=bias, L1=L1 if lr else None, L2=L2 if lr else None)
    pw = ref["w"]
    args = (to_dev(pw["packed"]), to_dev(pw["scale"]), to_dev(pw["zp"]) if asym else None)
    # exact accumulators on the oracle's own codes, through the split kernel
    qa = ref["a"]["q"] if bits == 8 else ref["a"]["packed"]
    acc = w4.w4_linear_cached_rot(to_dev(qa), to_dev(ref["a"]["scale"]),
                                  to_dev(ref["a"]["rowsum"].astype(np.int32)), bits, *args, out_i32=True)
    assert np.array_equal(np_(acc).astype(np.int64), ref["acc"])
    # the layer output with the GPU's own rotation and codes
    Xd = X.to(DEV)
    low = None
    if lr_mode == "x":
        low = w4.LowRank(l2=L2.to(DEV), x=Xd, l1=L1.t().contiguous().to(DEV))
    elif lr_mode == "t":
        low = w4.LowRank(l2=L2.to(DEV), t=w4.w4_lowrank_down(Xd, L1.t().contiguous().to(DEV)))
    q, s, rs = w4.w4_rotate_quant_act(Xd, g, bits)
    y = w4.w4_linear_cached_rot(q, s, rs, bits, *args, bias=bias.to(DEV), lowrank=low)
    err = rel_frob(y, ref["y64"])
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL
    if lr:
        assert rel_frob(torch.from_numpy(ref["y64"] - ref["lr"]), ref["y64"]) > 4 * FROB_TOL
    # w4_linear on the same shape takes the same split path (workspace sized for it)
    y2 = w4.w4_linear(Xd, g, bits, *args, bias=bias.to(DEV), lowrank=low)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


# --------------------------------------------------------------------------- exact ties
def _tie_rows_f32(M, K, g, bits, seed):
    """Rotated rows X' whose quotients by the token scale are exact half-integers, and the
    fp32 inputs X = X' . blockdiag(H_g / sqrt(g)) that produce them ((H_g / sqrt(g))^2 = I).
    Each row holds +-qmax once, so its scale is exactly 1; the other entries are multiples of
    1/2 inside (-qmax, qmax), most of them odd halves (ties)."""
    qmax = oracle.QMAX[bits]
    r = rng(seed)
    Xr = (r.integers(-2 * qmax + 1, 2 * qmax, size=(M, K)) | 1).astype(np.float64) / 2.0   # odd halves
    for m in range(M):
        Xr[m, r.integers(0, K)] = qmax if m % 2 == 0 else -qmax
    X = oracle.rotate(Xr, g)        # the rotation is its own inverse
    assert np.array_equal(X.astype(np.float32).astype(np.float64), X), "inputs must be exact in fp32"
    return torch.from_numpy(X.astype(np.float32)), Xr


def _tie_rows_bf16(M, K, g, bits, seed):
    """Like _tie_rows_f32, for bf16 inputs: a group of g holds either +-qmax alone or a few
    small half-integers whose signed sums all fit bf16's 8 significant bits."""
    qmax = oracle.QMAX[bits]
    r = rng(seed)
    Xr = np.zeros((M, K))
    for m in range(M):
        Xr[m, 0] = qmax if m % 2 == 0 else -qmax
        for grp in range(1, K // g):
            pos = r.choice(g, size=3, replace=False) + grp * g
            Xr[m, pos] = r.choice([-2.5, -1.5, -0.5, 0.5, 1.5, 2.5], size=3)
    X = oracle.rotate(Xr, g)
    Xb = torch.from_numpy(X.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(oracle.to_f64(Xb), X), "inputs must be exact in bf16"
    return Xb, Xr


@pytest.mark.parametrize("M,K,g,bits,dtype", [
    (16, 256, 64, 8, torch.float32), (9, 3072, 64, 4, torch.float32), (5, 4096, 64, 8, torch.float32),
    (40, 1024, 64, 4, torch.float32), (300, 512, 64, 8, torch.float32),
    (8, 3072, 256, 8, torch.bfloat16), (3, 12288, 256, 4, torch.bfloat16), (20, 1024, 64, 8, torch.bfloat16),
])
def test_rotate_quant_exact_ties_round_half_even(M, K, g, bits, dtype):
    """Crafted tokens whose rotated values over the token scale (exactly 1) sit exactly on
    half-integers: the GPU codes must equal the oracle's bit for bit, ties to even, with no
    tie allowance (both sides compute these values exactly)."""
    say("rotquant ties M=%d K=%d g=%d bits=%d %s" % (M, K, g, bits, dtype))
    make = _tie_rows_f32 if dtype == torch.float32 else _tie_rows_bf16
    X, Xr = make(M, K, g, bits, seed=M + K + bits)
    ref = oracle.rotate_quant_act(X, g, bits)
    assert np.array_equal(ref["rotated"], Xr) and np.all(ref["scale"] == 1.0)
    frac = np.abs(ref["pre"] - np.floor(ref["pre"]))
    n_ties = int((frac == 0.5).sum())
    say("  %d exact ties" % n_ties)
    assert n_ties >= M
    q, s, rs = w4.w4_rotate_quant_act(X.to(DEV), g, bits)
    assert np.all(np_(s) == 1.0)
    qg = np_(q)
    codes = oracle.unpack_nibbles(qg, signed=True) if bits == 4 else qg
    assert np.array_equal(codes.astype(np.int64), ref["q"].astype(np.int64))
    assert np.array_equal(np_(rs).astype(np.int64), ref["rowsum"])
    # half-even, not half-away: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2
    ties = frac == 0.5
    assert np.all(codes[ties] % 2 == 0)


def test_pack_weights_exact_ties():
    """Weight rows whose rotated values over the row scale (exactly 1) are half-integers: the
    packed bytes, scales and zero points equal the oracle's bit for bit.  Asymmetric rows with
    an odd zero point tell round-then-add-z from rounding after adding z; one row's zero point
    is itself a tie."""
    g, K = 64, 256
    say("pack ties K=%d g=%d" % (K, g))
    r = rng(77)
    sym = (r.integers(-13, 14, size=(6, K)) | 1).astype(np.float64) / 2.0   # odd halves in [-6.5, 6.5]
    for i in range(6):
        sym[i, r.integers(0, K)] = 7.0 if i % 2 else -7.0                   # scale exactly 1
    asym = np.zeros((6, K))
    for i, (lo, hi) in enumerate([(-5.0, 10.0), (-3.0, 12.0), (-7.0, 8.0), (-4.5, 10.5), (-1.0, 14.0),
                                  (-9.0, 6.0)]):
        row = (r.integers(int(2 * lo) + 1, int(2 * hi), size=K) | 1) / 2.0
        row = np.clip(row, lo + 0.5, hi - 0.5)
        row[0], row[1] = lo, hi                                             # (hi - lo) / 15 = 1
        asym[i] = row
    for rot, is_asym in ((sym, False), (asym, True)):
        W = oracle.rotate(rot, g)
        assert np.array_equal(W.astype(np.float32).astype(np.float64), W)
        Wt = torch.from_numpy(W.astype(np.float32))
        ref = oracle.pack_weights(Wt, g, is_asym)
        assert np.array_equal(ref["rotated"], rot) and np.all(ref["scale"] == 1.0)
        assert int((np.abs(ref["pre"] - np.floor(ref["pre"])) == 0.5).sum()) > K
        packed, s, zp = w4.w4_pack_weights(Wt.to(DEV), g, is_asym)
        assert np.array_equal(np_(packed), ref["packed"])
        assert np.array_equal(np_(s), ref["scale"])
        if is_asym:
            assert np.array_equal(np_(zp), ref["zp"])
            assert np.any(ref["zp"] % 2 == 1) and ref["zp"][3] == 4    # odd z; z = rint(4.5) = 4


# --------------------------------------------------------------------------- fused path vs oracle
@pytest.mark.parametrize("N,K,g,bits,asym,lr", [
    (1000, 8192, 64, 4, True, False),     # W4A4, g = 64, ragged N
    (520, 4096, 256, 4, False, True),     # W4A4 with the low-rank branch
    (4096, 12288, 256, 8, True, False),   # the text-encoder shape
    (300, 16384, 64, 8, False, False),
    (700, 3072, 256, 8, True, True),      # 12 waves per workgroup, one stage
])
def test_fused_single_token_matches_oracle(N, K, g, bits, asym, lr):
    """The one-launch path compared with the oracle directly: its int32 accumulators equal the
    oracle's GEMM of the (oracle-checked) activation codes, and its bf16 output is within the
    bar of the oracle's fp64 output."""
    say("fused vs oracle N=%d K=%d g=%d bits=%d asym=%s lr=%s" % (N, K, g, bits, asym, lr))
    assert w4.w4_linear_fused(1, N, K, g, bits)
    r = rng(N + K + g + bits)
    X = act_input(1, K, seed=N + 5 * K)
    W = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16)
    L1 = torch.from_numpy((r.standard_normal((K, 16)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    L2 = torch.from_numpy((r.standard_normal((16, N)) * 0.2).astype(np.float32)).to(torch.bfloat16)
    ref = oracle.linear(X, W, g, bits, asym, bias=bias, L1=L1 if lr else None, L2=L2 if lr else None)
    pw = ref["w"]
    args = (to_dev(pw["packed"]), to_dev(pw["scale"]), to_dev(pw["zp"]) if asym else None)
    Xd = X.to(DEV)
    low = w4.LowRank(l2=L2.to(DEV), x=Xd, l1=L1.t().contiguous().to(DEV)) if lr else None
    y = w4.w4_linear(Xd, g, bits, *args, bias=bias.to(DEV), lowrank=low)
    err = rel_frob(y, ref["y64"])
    say("  rel frob %.3e" % err)
    assert err <= FROB_TOL
    acc = np_(w4.w4_linear(Xd, g, bits, *args, out_i32=True)).astype(np.int64)
    q, _, _ = w4.w4_rotate_quant_act(Xd, g, bits)
    qg = np_(q)
    codes = oracle.unpack_nibbles(qg, signed=True) if bits == 4 else qg
    check_codes(codes, ref["a"]["q"], ref["a"]["pre"], "act codes")
    want = oracle.gemm_i64(codes.astype(np.int8), oracle.weight_operand(pw["packed"], pw["zp"], asym))
    assert np.array_equal(acc, want)


# --------------------------------------------------------------------------- rotate-quantize + low-rank
@pytest.mark.parametrize("M,K,g,bits,r", [
    (4608, 3072, 256, 8, 64),    # the DiT block input, QKV and MLP-up factors stacked
    (300, 3072, 256, 4, 32),
    (37, 4096, 64, 8, 20),       # ragged M and r
    (5, 1024, 256, 8, 16),       # fewer tokens than a block
    (129, 2048, 64, 4, 48),
    (40, 12288, 256, 8, 32),     # four waves per row
    (4608, 12288, 256, 8, 32),   # the DiT down-projection input
    (77, 8192, 64, 4, 64),       # two waves per row
    (3, 5120, 256, 8, 16),       # K = 5 x 1024 has no row-team split: two launches
])
def test_rotate_quant_lowrank_matches_oracle(M, K, g, bits, r):
    """One pass gives the same codes, scales and row sums as w4_rotate_quant_act (bit for bit)
    and t = X . L1 within fp32 rounding of the oracle's fp64 product; t can be a column range
    of a wider tensor (row stride)."""
    say("rotquant+lowrank M=%d K=%d g=%d bits=%d r=%d fused=%s" % (M, K, g, bits, r,
                                                                    w4.w4_rotate_quant_act_lowrank_fused(K, g)))
    X = act_input(M, K, seed=M + K + r)
    rg = rng(M + r)
    L1 = torch.from_numpy((rg.standard_normal((K, r)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    Xd = X.to(DEV)
    l1 = L1.t().contiguous().to(DEV)
    q, s, rs, t = w4.w4_rotate_quant_act_lowrank(Xd, g, bits, l1)
    q0, s0, rs0 = w4.w4_rotate_quant_act(Xd, g, bits)
    assert torch.equal(q, q0) and torch.equal(s.view(torch.int32), s0.view(torch.int32)) and torch.equal(rs, rs0)
    tref = oracle.to_f64(X) @ oracle.to_f64(L1)
    assert np.abs(np_(t) - tref).max() <= 1e-4 * np.abs(tref).max()
    # into columns [8, 8 + r) of a [M, r + 12] tensor
    wide = torch.full((M, r + 12), 7.0, dtype=torch.float32, device=DEV)
    w4.w4_rotate_quant_act_lowrank(Xd, g, bits, l1, t=wide[:, 8:8 + r])
    assert torch.equal(wide[:, 8:8 + r], t)
    assert bool((wide[:, :8] == 7.0).all()) and bool((wide[:, 8 + r:] == 7.0).all())
    if M >= 300:   # the codes against the oracle too
        ref = oracle.rotate_quant_act(X[:64], g, bits)
        qg = np_(q)[:64]
        codes = oracle.unpack_nibbles(qg, signed=True) if bits == 4 else qg
        check_codes(codes, ref["q"], ref["pre"], "act codes")
