"""w4_linear_noalloc: the whole layer with the library's per-device scratch array instead of a
caller workspace (for callers that cannot allocate).  Its output must equal w4_linear's.
Two calls in a row, the second smaller, so the second call runs on the scratch the first one
left behind."""
import numpy as np
import pytest
import torch

import int4_weight_quantized_block_amd as w4
from parity import FROB_TOL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def case(M, N, K, seed, lr_rank=0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    X = torch.randn(M, K, generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn(N, K, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    bias = (torch.randn(N, generator=g, device=DEV) * 0.01).to(torch.bfloat16)
    low = None
    if lr_rank:
        l1 = (torch.randn(lr_rank, K, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
        l2 = (torch.randn(lr_rank, N, generator=g, device=DEV) * 0.2).to(torch.bfloat16)
        low = w4.LowRank(l2=l2, x=X, l1=l1)
    return X, W, bias, low


@pytest.mark.parametrize("shapes", [
    # (M, N, K, g, bits, asym, lr_rank): large-M GEMM then the K-split small-M path
    [(2048, 3072, 3072, 256, 8, False, 32), (40, 3072, 3072, 256, 4, True, 16)],
    # K-split (partials in the scratch) then the one-token fused launch
    [(24, 4096, 12288, 256, 8, True, 0), (1, 4096, 12288, 256, 8, True, 0)],
    # W4A4 with the low-rank t in the scratch, then a smaller W4A8 with a streaming kernel
    [(700, 1536, 4096, 64, 4, False, 32), (9, 1000, 2048, 64, 8, False, 8)],
])
def test_noalloc_equals_w4_linear_two_calls(shapes):
    for i, (M, N, K, gsz, bits, asym, rank) in enumerate(shapes):
        say("noalloc call %d: M=%d N=%d K=%d g=%d bits=%d asym=%s r=%d" % (i, M, N, K, gsz, bits, asym, rank))
        X, W, bias, low = case(M, N, K, seed=M + N + K + i, lr_rank=rank)
        packed, s_w, zp = w4.w4_pack_weights(W, gsz, asym)
        ref = w4.w4_linear(X, gsz, bits, packed, s_w, zp, bias=bias, lowrank=low)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        y = w4.w4_linear_noalloc(X, gsz, bits, packed, s_w, zp, bias=bias, lowrank=low, out=out)
        torch.cuda.synchronize()
        assert y.data_ptr() == out.data_ptr()
        if torch.equal(y.view(torch.int16), ref.view(torch.int16)):
            say("  bit-identical to w4_linear")
        else:
            # only a low-rank shape whose split partials do not fit the scratch may differ, and
            # only within the bf16 bar
            assert low is not None
            err = ((y.float() - ref.float()).norm() / ref.float().norm()).item()
            say("  rel frob vs w4_linear %.3e" % err)
            assert err <= FROB_TOL
        a_ref = w4.w4_linear(X, gsz, bits, packed, s_w, zp, out_i32=True)
        a = w4.w4_linear_noalloc(X, gsz, bits, packed, s_w, zp, out_i32=True)
        assert torch.equal(a, a_ref)


def test_noalloc_rejects_calls_past_the_scratch():
    limit = w4.w4_noalloc_scratch_bytes()
    assert limit == 64 << 20
    M, K, N = 8192, 8192, 64       # 64 MiB of int8 codes plus scales: past the limit
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    packed = torch.zeros((N, K // 2), dtype=torch.uint8, device=DEV)
    s_w = torch.ones(N, dtype=torch.float32, device=DEV)
    with pytest.raises(w4.W4Error) as e:
        w4.w4_linear_noalloc(X, 256, 8, packed, s_w)
    assert e.value.status == w4.W4_ERR_WORKSPACE
    # W4A4 codes of the same input take half: they fit
    y = w4.w4_linear_noalloc(X, 256, 4, packed, s_w)
    torch.cuda.synchronize()
    assert not bool(y.float().abs().sum())
