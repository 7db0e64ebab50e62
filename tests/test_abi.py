"""Host-side checks of the C-ABI library and its binding (no GPU needed, no kernel launched).

- every function that include/w4.h declares is exported by libw4.so and bound in Python;
- argument validation rejects bad calls with the documented status code before anything is
  launched (fake, never dereferenced pointers; the calls return before any HIP work);
- workspace sizes, status strings, the per-thread error message;
- the rotation cache's keying (hit / miss rules) with the activation call stubbed out.
"""
import ctypes
import os
import re

import pytest
import torch

import int4_weight_quantized_block_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")
A = 0x10000      # a 16-byte aligned fake device address (never dereferenced)
U = 0x10008      # not 16-byte aligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.library_path()):
        from int4_weight_quantized_block_amd import build
        build.build()
    return w4.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(w4_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls_and_helpers():
    names = declared_functions()
    for n in ["w4_pack_weights", "w4_rotate_quant_act", "w4_linear", "w4_linear_cached_rot",
              "w4_workspace_bytes", "w4_status_string", "w4_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
        assert n in w4.EXPORTS, "binding lacks " + n


def test_status_strings_and_version(lib):
    expect = ["W4_OK", "W4_ERR_INVALID_ARG", "W4_ERR_SHAPE", "W4_ERR_UNSUPPORTED", "W4_ERR_ALIGN",
              "W4_ERR_HIP", "W4_ERR_WORKSPACE"]
    for code, name in enumerate(expect):
        assert lib.w4_status_string(code).decode() == name
    assert lib.w4_status_string(99).decode() == "W4_ERR_UNKNOWN"
    assert b"gfx950" in lib.w4_version()


def test_workspace_sizes(lib):
    assert lib.w4_workspace_bytes(0, 8, 256, 8, 32) == 0
    assert lib.w4_workspace_bytes(100, 8, 256, 8, 32) == 12800
    assert lib.w4_workspace_bytes(3, 8, 256, 8, 5) == 256          # rounded up to 256 bytes
    # q (int8 [M, K]) + token scales + token rowsums, each 256-byte aligned (+ low-rank t)
    assert lib.w4_linear_workspace_bytes(100, 8, 256, 8, 0) == 25600 + 512 + 512
    assert lib.w4_linear_workspace_bytes(100, 8, 256, 4, 0) == 12800 + 512 + 512
    assert lib.w4_linear_workspace_bytes(100, 8, 256, 8, 32) == 25600 + 1024 + 12800
    # large M: partial sums only when the 256 x 192 tiles leave a tail of at most a quarter
    # round of the 256 compute units (the count this host reports when it has no GPU)
    tile = 256 * 192 * 4
    assert lib.w4_workspace_bytes(4096, 3072, 3072, 8, 0) == 0            # 256 tiles: whole rounds
    assert lib.w4_workspace_bytes(4608, 3072, 3072, 8, 0) == 32 * 8 * tile  # 288 = 256 + 32, 8 K ranges
    assert lib.w4_workspace_bytes(4608, 9216, 3072, 8, 0) == 0            # tail of 96: one pass
    assert lib.w4_workspace_bytes(4608, 3072, 3008, 8, 0) == 0            # K % 128 != 0: one pass


def pack(lib, W=A, dt=w4.W4_BF16, N=8, K=256, g=64, mode=w4.W4_SYM, packed=A, scale=A, zp=None):
    return lib.w4_pack_weights(W, dt, N, K, g, mode, packed, scale, zp, None)


def test_pack_weights_validation(lib):
    assert pack(lib, g=128) == w4.W4_ERR_UNSUPPORTED
    assert pack(lib, K=320, g=256) == w4.W4_ERR_SHAPE
    assert pack(lib, K=64 * 513 * 2) == w4.W4_ERR_SHAPE          # K > W4_MAX_K
    assert pack(lib, dt=7) == w4.W4_ERR_INVALID_ARG
    assert pack(lib, mode=3) == w4.W4_ERR_INVALID_ARG
    assert pack(lib, N=0) == w4.W4_ERR_SHAPE
    assert pack(lib, W=None) == w4.W4_ERR_INVALID_ARG
    assert pack(lib, W=U) == w4.W4_ERR_ALIGN
    assert pack(lib, zp=A) == w4.W4_ERR_INVALID_ARG               # zero points only for W4_ASYM
    assert pack(lib, mode=w4.W4_ASYM, zp=None) == w4.W4_ERR_INVALID_ARG
    assert b"w4_pack_weights" in lib.w4_last_error()


def rq(lib, X=A, dt=w4.W4_BF16, M=4, K=256, g=64, bits=8, q=A, s=A, r=A):
    return lib.w4_rotate_quant_act(X, dt, M, K, g, bits, q, s, r, None)


def test_rotate_quant_act_validation(lib):
    assert rq(lib, bits=5) == w4.W4_ERR_UNSUPPORTED
    assert rq(lib, g=32) == w4.W4_ERR_UNSUPPORTED
    assert rq(lib, M=-1) == w4.W4_ERR_SHAPE
    assert rq(lib, K=200) == w4.W4_ERR_SHAPE
    assert rq(lib, q=None) == w4.W4_ERR_INVALID_ARG
    assert rq(lib, s=U) == w4.W4_ERR_ALIGN
    assert rq(lib, M=0, X=None) == w4.W4_OK                       # M = 0 is a no-op
    assert lib.w4_last_error() == b""


def cached(lib, M=100, N=64, K=256, bits=8, y_kind=w4.W4_OUT_BF16, lr=None, ws=None, ws_bytes=0, q=A,
           bias=None, bias_dtype=w4.W4_BF16, zp=None):
    return lib.w4_linear_cached_rot(q, A, A, bits, A, A, zp, bias, bias_dtype, lr, M, N, K, A, y_kind, ws,
                                    ws_bytes, None)


def test_linear_cached_rot_validation(lib):
    assert cached(lib, bits=2) == w4.W4_ERR_UNSUPPORTED
    assert cached(lib, K=100) == w4.W4_ERR_SHAPE
    assert cached(lib, N=0) == w4.W4_ERR_SHAPE
    assert cached(lib, y_kind=5) == w4.W4_ERR_INVALID_ARG
    assert cached(lib, q=None) == w4.W4_ERR_INVALID_ARG
    assert cached(lib, zp=U) == w4.W4_ERR_ALIGN
    assert cached(lib, bias=A, bias_dtype=9) == w4.W4_ERR_INVALID_ARG
    lr = w4._LowRankC(A, A, None, A, 0)
    assert cached(lib, lr=ctypes.byref(lr)) == w4.W4_ERR_UNSUPPORTED        # rank 0
    lr = w4._LowRankC(A, A, None, None, 16)
    assert cached(lib, lr=ctypes.byref(lr)) == w4.W4_ERR_INVALID_ARG        # no L2
    lr = w4._LowRankC(A, A, None, A, 16)                                    # t computed in the workspace
    assert cached(lib, lr=ctypes.byref(lr), ws=A, ws_bytes=100) == w4.W4_ERR_WORKSPACE
    assert cached(lib, M=0) == w4.W4_OK


def test_linear_cached_rot_multi_validation(lib):
    """Every output is checked before anything is launched; a low-rank branch must give t."""
    def outs(n=2, **kw):
        arr = (w4._LinearOutC * n)()
        for i in range(n):
            o = arr[i]
            o.packed, o.row_scale, o.zp, o.bias, o.bias_dtype = A, A, None, None, w4.W4_BF16
            o.N, o.Y, o.y_kind = 64, A, w4.W4_OUT_BF16
        for k, v in kw.items():
            setattr(arr[n - 1], k, v)
        return arr

    def multi(arr, count=None, M=100, K=256, bits=8, q=A):
        n = len(arr) if count is None else count
        return lib.w4_linear_cached_rot_multi(q, A, A, bits, M, K, n, arr, None, 0, None)

    assert multi(outs(), count=0) == w4.W4_ERR_INVALID_ARG
    assert multi(outs(9)) == w4.W4_ERR_INVALID_ARG                           # more than W4_MULTI_MAX
    assert lib.w4_linear_cached_rot_multi(A, A, A, 8, 100, 256, 2, None, None, 0, None) == w4.W4_ERR_INVALID_ARG
    assert multi(outs(), bits=2) == w4.W4_ERR_UNSUPPORTED
    assert multi(outs(), K=100) == w4.W4_ERR_SHAPE
    assert multi(outs(N=0)) == w4.W4_ERR_SHAPE                                # the second output
    assert multi(outs(y_kind=7)) == w4.W4_ERR_INVALID_ARG
    assert multi(outs(zp=U)) == w4.W4_ERR_ALIGN
    assert multi(outs(Y=None)) == w4.W4_ERR_INVALID_ARG
    assert multi(outs(bias=A, bias_dtype=5)) == w4.W4_ERR_INVALID_ARG
    assert multi(outs(), q=None) == w4.W4_ERR_INVALID_ARG
    lr = w4._LowRankC(A, A, None, A, 16)                                     # x and l1 but no t
    assert multi(outs(lr=ctypes.pointer(lr))) == w4.W4_ERR_INVALID_ARG
    lr = w4._LowRankC(None, None, U, A, 16)
    assert multi(outs(lr=ctypes.pointer(lr))) == w4.W4_ERR_ALIGN
    lr = w4._LowRankC(None, None, A, A, 65)
    assert multi(outs(lr=ctypes.pointer(lr))) == w4.W4_ERR_UNSUPPORTED
    lr = w4._LowRankC(None, None, A, A, 16, 8)                               # ldt < r
    assert multi(outs(lr=ctypes.pointer(lr))) == w4.W4_ERR_INVALID_ARG
    assert multi(outs(), M=0) == w4.W4_OK


def test_linear_validation(lib):
    def lin(M=100, K=256, g=64, ws=A, ws_bytes=0, Y=A, x_dtype=w4.W4_BF16):
        return lib.w4_linear(A, x_dtype, M, K, g, 8, A, A, None, None, w4.W4_BF16, None, 64, Y, w4.W4_OUT_BF16,
                             ws, ws_bytes, None)
    need = lib.w4_linear_workspace_bytes(100, 64, 256, 8, 0)
    assert lin(ws_bytes=need - 1) == w4.W4_ERR_WORKSPACE
    assert lin(ws=None, ws_bytes=need) == w4.W4_ERR_WORKSPACE
    assert lin(ws=U, ws_bytes=need) == w4.W4_ERR_ALIGN
    assert lin(Y=None, ws_bytes=need) == w4.W4_ERR_INVALID_ARG              # caught before any launch
    assert lin(g=32) == w4.W4_ERR_UNSUPPORTED                               # not a rotation size
    assert lin(x_dtype=4) == w4.W4_ERR_INVALID_ARG
    assert lin(M=0, ws=None) == w4.W4_OK


def test_linear_noalloc_validation(lib):
    """The no-workspace entry point checks everything before it looks up its scratch array
    (so none of these calls touches a device)."""
    def na(M=100, K=256, g=64, bits=8, Y=A, x_dtype=w4.W4_BF16, lr=None, N=64, X=A):
        return lib.w4_linear_noalloc(X, x_dtype, M, K, g, bits, A, A, None, None, w4.W4_BF16, lr, N, Y,
                                     w4.W4_OUT_BF16, None)
    assert lib.w4_noalloc_scratch_bytes() == 64 << 20
    assert na(M=8192, K=8192) == w4.W4_ERR_WORKSPACE                       # 64 MiB of int8 codes + scales
    assert b"limit" in lib.w4_last_error()
    lr = w4._LowRankC(A, A, None, A, 64)                                   # t of 64 ranks on top of the codes
    assert na(M=8000, K=8192, lr=ctypes.byref(lr)) == w4.W4_ERR_WORKSPACE
    assert na(Y=None) == w4.W4_ERR_INVALID_ARG
    assert na(X=U) == w4.W4_ERR_ALIGN
    assert na(g=32) == w4.W4_ERR_UNSUPPORTED
    assert na(bits=3) == w4.W4_ERR_UNSUPPORTED
    assert na(x_dtype=4) == w4.W4_ERR_INVALID_ARG
    assert na(N=0) == w4.W4_ERR_SHAPE
    assert na(M=0, X=None) == w4.W4_OK


def test_grouped_validation(lib):
    """The grouped-scale calls check rotation size, group width, bit width and shapes before
    anything is launched."""
    def pg(N=8, K=256, g=64, gw=64, W=A, packed=A, gs=A):
        return lib.w4_pack_weights_grouped(W, w4.W4_BF16, N, K, g, gw, packed, gs, None)
    assert pg(gw=48) == w4.W4_ERR_UNSUPPORTED
    assert pg(gw=16) == w4.W4_ERR_UNSUPPORTED
    assert pg(K=288, gw=32) == w4.W4_ERR_SHAPE                             # K not a multiple of 64
    assert pg(g=128) == w4.W4_ERR_UNSUPPORTED
    assert pg(K=1024, g=4096) == w4.W4_ERR_SHAPE                           # K < g
    assert pg(gs=None) == w4.W4_ERR_INVALID_ARG
    assert pg(packed=U) == w4.W4_ERR_ALIGN

    def lg(M=100, K=256, g=64, bits=8, gw=64, Y=A, ws=A, ws_bytes=1 << 20, x_dtype=w4.W4_BF16, y_kind=w4.W4_OUT_BF16):
        return lib.w4_linear_grouped(A, x_dtype, M, K, g, bits, A, A, gw, None, w4.W4_BF16, None, 64, Y, y_kind,
                                     ws, ws_bytes, None)
    assert lg(bits=16) == w4.W4_ERR_UNSUPPORTED                             # W4A16 with a rotation
    assert lg(bits=16, g=0, x_dtype=w4.W4_F32) == w4.W4_ERR_UNSUPPORTED
    assert lg(bits=16, g=0, y_kind=w4.W4_OUT_I32) == w4.W4_ERR_INVALID_ARG
    assert lg(g=0) == w4.W4_ERR_UNSUPPORTED                                 # integer codes need a rotation
    assert lg(bits=2) == w4.W4_ERR_UNSUPPORTED
    assert lg(gw=512) == w4.W4_ERR_UNSUPPORTED
    assert lg(ws_bytes=10) == w4.W4_ERR_WORKSPACE
    assert lg(Y=None) == w4.W4_ERR_INVALID_ARG
    assert lg(M=0, ws=None, ws_bytes=0) == w4.W4_OK
    need = lib.w4_linear_grouped_workspace_bytes(100, 64, 256, 8, 64, 0)
    assert need == 100 * 256 + 2 * 512                                      # codes, token scales, row sums
    assert lib.w4_linear_grouped_workspace_bytes(100, 64, 256, 16, 64, 0) == 0
    assert lib.w4_grouped_workspace_bytes(100, 64, 256, 8, 64, 32) == 100 * 32 * 4

    def cg(M=100, K=256, bits=8, gw=64, q=A, s=A):
        return lib.w4_linear_cached_rot_grouped(q, s, bits, A, A, gw, None, w4.W4_BF16, None, M, 64, K, A,
                                                w4.W4_OUT_BF16, None, 0, None)
    assert cg(bits=16) == w4.W4_ERR_UNSUPPORTED
    assert cg(s=None) == w4.W4_ERR_INVALID_ARG
    assert cg(K=320, gw=128) == w4.W4_ERR_SHAPE
    assert cg(M=0) == w4.W4_OK


def test_probe_library_is_separate_and_validates():
    """The measurement probes live in libw4probe.so (include/w4_probe.h), not in the layer's
    library; invalid arguments return 1 before anything is launched."""
    probe_h = os.path.join(ROOT, "include", "w4_probe.h")
    text = re.sub(r"/\*.*?\*/", "", open(probe_h).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(w4_probe_\w+)\s*\(", text)))
    assert names == ["w4_probe_mfma_rate", "w4_probe_read_rate"]
    main = w4.load_library()
    assert not any(hasattr(main, n) for n in names)
    path = os.path.join(os.path.dirname(w4.library_path()), "libw4probe.so")
    if not os.path.exists(path):
        from int4_weight_quantized_block_amd import build
        build.build()
    P = ctypes.CDLL(path)
    P.w4_probe_mfma_rate.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.w4_probe_read_rate.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert P.w4_probe_mfma_rate(0, 10, 1, A, None) == 1
    assert P.w4_probe_mfma_rate(8, 0, 1, A, None) == 1
    assert P.w4_probe_mfma_rate(8, 10, 1, None, None) == 1
    assert P.w4_probe_read_rate(A, 100, 8, A, None) == 1        # not a multiple of 16
    assert P.w4_probe_read_rate(U, 1024, 8, A, None) == 1
    assert P.w4_probe_read_rate(A, 1024, 0, A, None) == 1


def test_error_message_is_per_thread(lib):
    import threading
    assert pack(lib, g=128) == w4.W4_ERR_UNSUPPORTED
    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.w4_last_error()))
    t.start()
    t.join()
    assert seen == [b""]
    assert b"g=128" in lib.w4_last_error()


def test_rotation_cache_keys(monkeypatch):
    calls = []

    def fake(X, g, bits):
        calls.append((X.data_ptr(), g, bits))
        return ("codes", len(calls))

    monkeypatch.setattr(w4, "w4_rotate_quant_act", fake)
    c = w4.RotationCache()
    x = torch.zeros(8, 256, dtype=torch.bfloat16)
    a = c.get(x, 256, 8)
    assert c.get(x, 256, 8) is a and c.hits == 1 and c.misses == 1       # same input, same g, bits
    c.get(x, 64, 8)
    c.get(x, 256, 4)
    assert c.misses == 3                                                   # g and act_bits are part of the key
    x.add_(1)                                                              # in-place update: new version
    assert c.get(x, 256, 8) is not a and c.misses == 4
    c.get(x[:4], 256, 8)                                                   # a view of a different shape
    c.get(x[4:], 256, 8)                                                   # a view at another offset
    assert c.misses == 6
    assert len(c) == 6
    c.clear()
    assert len(c) == 0


def test_linear_fused_query(lib):
    """w4_linear runs fused only for one bf16 token with K in whole 3072-k stages up to 12288 or
    whole 2048-k stages up to 16384, and N within one workgroup of up to 32 rows per compute
    unit (256 on MI355X, the default without a GPU)."""
    bf, f32 = w4.W4_BF16, w4.W4_F32
    assert lib.w4_linear_fused(1, 4096, 12288, 256, 8, bf) == 1
    assert lib.w4_linear_fused(1, 4096, 16384, 64, 4, bf) == 1
    assert lib.w4_linear_fused(1, 4096, 12288, 256, 8, f32) == 0      # fp32 input
    assert lib.w4_linear_fused(2, 4096, 4096, 256, 8, bf) == 0        # two tokens
    assert lib.w4_linear_fused(1, 8192, 4096, 256, 8, bf) == 1        # 32 rows per workgroup
    assert lib.w4_linear_fused(1, 8193, 4096, 256, 8, bf) == 0        # more than one workgroup per CU
    assert lib.w4_linear_fused(1, 4096, 3072, 256, 8, bf) == 1        # one 3072-k stage (12 waves)
    assert lib.w4_linear_fused(1, 4096, 1024, 256, 8, bf) == 0        # neither stage size
    assert lib.w4_linear_fused(1, 4096, 15360, 256, 8, bf) == 0       # 3072-k stages past 12288
    assert lib.w4_linear_fused(1, 4096, 18432, 256, 8, bf) == 0       # K past 16384
    assert lib.w4_linear_fused(1, 4096, 4096, 128, 8, bf) == 0        # unsupported g
    assert lib.w4_linear_fused(1, 4096, 4096, 256, 5, bf) == 0        # unsupported bits
    assert lib.w4_linear_fused(1, 4096, 4096, 256, 8, 7) == 0         # unknown dtype
    assert w4.w4_linear_fused(1, 4096, 12288, 256, 8) is True


def _bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_binding_rejects_mis_shaped_tensors_before_launch():
    """The C ABI cannot see sizes, so the binding checks every tensor against (M, N, K, r);
    these CPU tensors never reach the device check or the library."""
    M, N, K, r = 8, 64, 256, 4
    i8 = lambda *s: torch.zeros(*s, dtype=torch.int8)
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    good = dict(q=i8(M, K), tok_scale=f32(M), tok_rowsum=i32(M), act_bits=8, packed=u8(N, K // 2),
                row_scale=f32(N))
    bad_cases = [
        dict(q=i8(M, K // 2)),                       # A8 codes must be [M, K]
        dict(q=u8(M, K), act_bits=4),                # A4 codes must be [M, K/2]
        dict(tok_scale=f32(M - 1)),
        dict(tok_rowsum=i32(M + 1)),
        dict(row_scale=f32(N - 1)),
        dict(zp=u8(N - 1)),
        dict(bias=_bf(N - 1)),
        dict(bias=_bf(1, N)),
        dict(q=i8(M * K)),                           # not 2-D
        dict(lowrank=w4.LowRank(l2=_bf(r, N - 1), t=f32(M, r))),
        dict(lowrank=w4.LowRank(l2=_bf(r, N), t=f32(M, r + 1))),
        dict(lowrank=w4.LowRank(l2=_bf(r, N), x=_bf(M, K - 2), l1=_bf(r, K))),
        dict(lowrank=w4.LowRank(l2=_bf(r, N), x=_bf(M, K), l1=_bf(r + 1, K))),
        dict(lowrank=w4.LowRank(l2=_bf(r, N))),      # neither t nor (x, l1)
        dict(out=torch.zeros(M, N + 1, dtype=torch.bfloat16)),
    ]
    for bad in bad_cases:
        kw = dict(good)
        kw.update(bad)
        with pytest.raises(ValueError):
            w4.w4_linear_cached_rot(**kw)
    # the whole layer: X [M, K] against packed [N, K/2]
    with pytest.raises(ValueError):
        w4.w4_linear(_bf(M, K + 2), 64, 8, u8(N, K // 2), f32(N))
    with pytest.raises(ValueError):
        w4.w4_linear(_bf(M, K), 64, 8, u8(N, K // 2), f32(N), bias=f32(N + 3))
    with pytest.raises(ValueError):
        w4.w4_linear(_bf(M, K), 64, 8, u8(N, K // 2), f32(N),
                     lowrank=w4.LowRank(l2=_bf(r, N), x=_bf(M + 1, K), l1=_bf(r, K)))
    with pytest.raises(ValueError):
        w4.w4_lowrank_down(_bf(M, K), _bf(r, K - 8))
    with pytest.raises(ValueError):
        w4.w4_rotate_quant_act(_bf(K), 64, 8)
    with pytest.raises(ValueError):
        w4.w4_pack_weights(_bf(N, K, 1), 64)
    # well-shaped CPU tensors get past the shape checks and stop at the device check
    with pytest.raises(ValueError, match="GPU tensor"):
        w4.w4_linear_cached_rot(**good)
    # several linears on the same codes: every output is checked against (M, N_i, K)
    o = lambda **kw: w4.LinearOut(**dict(dict(packed=u8(N, K // 2), row_scale=f32(N)), **kw))
    codes = dict(q=i8(M, K), tok_scale=f32(M), tok_rowsum=i32(M), act_bits=8)
    for bad in ([o(), o(packed=u8(N, K))],                  # another K
                [o(), o(row_scale=f32(N + 1))],
                [o(bias=_bf(N - 1))],
                [o(lowrank=w4.LowRank(l2=_bf(r, N), x=_bf(M, K), l1=_bf(r, K)))],   # no t
                [o(lowrank=w4.LowRank(l2=_bf(r, N), t=f32(M + 1, r)))],
                [o(out=torch.zeros(M, N - 1, dtype=torch.bfloat16))],
                [], [o()] * 9):
        with pytest.raises(ValueError):
            w4.w4_linear_cached_rot_multi(outs=bad, **codes)
    with pytest.raises(ValueError, match="GPU tensor"):
        w4.w4_linear_cached_rot_multi(outs=[o(), o()], **codes)


def test_rotation_cache_key_includes_stream(monkeypatch):
    calls = []
    monkeypatch.setattr(w4, "w4_rotate_quant_act", lambda X, g, b: calls.append(1) or ("codes", len(calls)))
    stream = [11]
    monkeypatch.setattr(w4.RotationCache, "_stream_of", staticmethod(lambda X: stream[0]))
    c = w4.RotationCache()
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    a = c.get(x, 256, 8)
    assert c.get(x, 256, 8) is a and c.hits == 1
    stream[0] = 12                                   # the same input looked up from another stream
    b = c.get(x, 256, 8)
    assert b is not a and c.misses == 2


def test_out_buffer_writes_bump_the_version(monkeypatch):
    """A linear writing into out= bumps its version, so a cache keyed on it recomputes."""
    class FakeLib:
        def __getattr__(self, name):
            return lambda *a: 0 if name.startswith("w4_linear") else 0
    monkeypatch.setattr(w4, "load_library", lambda: FakeLib())
    monkeypatch.setattr(w4, "_dev", lambda t, name, dtypes: 0)
    monkeypatch.setattr(w4, "_stream", lambda d: 0)
    monkeypatch.setattr(w4, "w4_linear_workspace_bytes", lambda *a: 0)
    monkeypatch.setattr(w4, "w4_workspace_bytes", lambda *a: 0)
    M, N, K = 4, 16, 256
    out = torch.zeros(M, N, dtype=torch.bfloat16)
    v0 = out._version
    w4.w4_linear(_bf(M, K), 64, 8, torch.zeros(N, K // 2, dtype=torch.uint8), torch.zeros(N), out=out)
    assert out._version == v0 + 1
    w4.w4_linear_cached_rot(torch.zeros(M, K, dtype=torch.int8), torch.zeros(M), torch.zeros(M, dtype=torch.int32),
                            8, torch.zeros(N, K // 2, dtype=torch.uint8), torch.zeros(N), out=out)
    assert out._version == v0 + 2


def test_phase_probe_anchors_occur_once():
    # the GEMM phase probe instruments a copy of gemm.hip at fixed anchor strings; each must
    # occur exactly once, or the probe would stamp the wrong place (checked on the host; the
    # probe itself is built and run only for measurement)
    from int4_weight_quantized_block_amd import phase_probe
    src = open(os.path.join(ROOT, "int4_weight_quantized_block_amd", "csrc", "gemm.hip")).read()
    for anchor, _ in phase_probe._EDITS:
        assert src.count(anchor) == 1, anchor
