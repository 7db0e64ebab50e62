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


def test_linear_validation(lib):
    def lin(M=100, K=256, g=64, ws=A, ws_bytes=0, Y=A, x_dtype=w4.W4_BF16):
        return lib.w4_linear(A, x_dtype, M, K, g, 8, A, A, None, None, w4.W4_BF16, None, 64, Y, w4.W4_OUT_BF16,
                             ws, ws_bytes, None)
    need = lib.w4_linear_workspace_bytes(100, 64, 256, 8, 0)
    assert lin(ws_bytes=need - 1) == w4.W4_ERR_WORKSPACE
    assert lin(ws=None, ws_bytes=need) == w4.W4_ERR_WORKSPACE
    assert lin(ws=U, ws_bytes=need) == w4.W4_ERR_ALIGN
    assert lin(Y=None, ws_bytes=need) == w4.W4_ERR_INVALID_ARG              # caught before any launch
    assert lin(g=16) == w4.W4_ERR_UNSUPPORTED
    assert lin(x_dtype=4) == w4.W4_ERR_INVALID_ARG
    assert lin(M=0, ws=None) == w4.W4_OK


def test_probe_validation(lib):
    assert lib.w4_probe_mfma_rate(0, 10, 1, A, None) == w4.W4_ERR_INVALID_ARG
    assert lib.w4_probe_mfma_rate(8, 0, 1, A, None) == w4.W4_ERR_INVALID_ARG
    assert lib.w4_probe_mfma_rate(8, 10, 1, None, None) == w4.W4_ERR_INVALID_ARG


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
    """w4_linear runs fused only for one bf16 token with K <= 16384 in whole 2048-k stages and
    N within one workgroup of up to 32 rows per compute unit (256 on MI355X, the default
    without a GPU)."""
    bf, f32 = w4.W4_BF16, w4.W4_F32
    assert lib.w4_linear_fused(1, 4096, 12288, 256, 8, bf) == 1
    assert lib.w4_linear_fused(1, 4096, 16384, 64, 4, bf) == 1
    assert lib.w4_linear_fused(1, 4096, 12288, 256, 8, f32) == 0      # fp32 input
    assert lib.w4_linear_fused(2, 4096, 4096, 256, 8, bf) == 0        # two tokens
    assert lib.w4_linear_fused(1, 8192, 4096, 256, 8, bf) == 1        # 32 rows per workgroup
    assert lib.w4_linear_fused(1, 8193, 4096, 256, 8, bf) == 0        # more than one workgroup per CU
    assert lib.w4_linear_fused(1, 4096, 3072, 256, 8, bf) == 0        # not whole 2048-k stages
    assert lib.w4_linear_fused(1, 4096, 18432, 256, 8, bf) == 0       # K past 16384
    assert lib.w4_linear_fused(1, 4096, 4096, 128, 8, bf) == 0        # unsupported g
    assert lib.w4_linear_fused(1, 4096, 4096, 256, 5, bf) == 0        # unsupported bits
    assert lib.w4_linear_fused(1, 4096, 4096, 256, 8, 7) == 0         # unknown dtype
    assert w4.w4_linear_fused(1, 4096, 12288, 256, 8) is True
