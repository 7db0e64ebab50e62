"""The rotate-quantize + linear pair captured in a HIP graph (as bench.py times it) gives the
same bytes as eager launches, on every replay, with eager work on the same stream between the
replays.  The library's calls enqueue kernels only (no memset, no allocation), so they can be
captured."""
import numpy as np
import pytest
import torch

import int4_weight_quantized_block_amd as w4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("M,N,K,bits", [(300, 384, 1024, 8), (40, 256, 3072, 4), (8, 512, 4096, 8),
                                         (4608, 3072, 3072, 8)])  # the last: split tail (3 launches)
def test_graph_replay_matches_eager(M, N, K, bits):
    say("graph replay M=%d N=%d K=%d bits=%d" % (M, N, K, bits))
    g = torch.Generator().manual_seed(M + N + K)
    X = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    W = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    bias = (torch.randn(N, generator=g) * 0.01).to(torch.bfloat16).to(DEV)
    packed, s_w, _ = w4.w4_pack_weights(W, 256, False)
    q, sx, rs = w4.w4_rotate_quant_act(X, 256, bits)
    ws_bytes = w4.load_library().w4_workspace_bytes(M, N, K, bits, 0)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    y_eager = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, bias=bias, ws=ws)
    torch.cuda.synchronize()

    q2, sx2, rs2 = torch.empty_like(q), torch.empty_like(sx), torch.empty_like(rs)
    y2 = torch.empty_like(y_eager)
    L = w4.load_library()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        st = torch.cuda.current_stream().cuda_stream
        w4._check(L.w4_rotate_quant_act(X.data_ptr(), w4.W4_BF16, M, K, 256, bits, q2.data_ptr(), sx2.data_ptr(),
                                        rs2.data_ptr(), st))
        w4._check(L.w4_linear_cached_rot(q2.data_ptr(), sx2.data_ptr(), rs2.data_ptr(), bits, packed.data_ptr(),
                                         s_w.data_ptr(), None, bias.data_ptr(), w4.W4_BF16, None, M, N, K,
                                         y2.data_ptr(), w4.W4_OUT_BF16, ws.data_ptr(), ws_bytes, st))
    for rep in range(3):
        y2.fill_(0)
        q2.fill_(0)
        _ = w4.w4_linear_cached_rot(q, sx, rs, bits, packed, s_w, bias=bias, ws=ws)  # eager work between
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(q2, q), rep
        assert torch.equal(sx2, sx) and torch.equal(rs2, rs), rep
        assert torch.equal(y2.view(torch.int16), y_eager.view(torch.int16)), rep


@pytest.mark.parametrize("N,K,asym", [(4096, 12288, True), (1000, 4096, False)])
def test_graph_replay_fused_single_token(N, K, asym):
    """w4_linear at one token (the fused rotate + quantize + GEMM launch) captured in a graph:
    every replay equals the eager result, with eager work on the stream between replays."""
    say("graph replay fused N=%d K=%d asym=%s" % (N, K, asym))
    assert w4.w4_linear_fused(1, N, K, 256, 8)
    g = torch.Generator().manual_seed(N + K)
    X = torch.randn(1, K, generator=g).to(torch.bfloat16).to(DEV)
    W = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    bias = (torch.randn(N, generator=g) * 0.01).to(torch.bfloat16).to(DEV)
    packed, s_w, zp = w4.w4_pack_weights(W, 256, asym)
    y_eager = w4.w4_linear(X, 256, 8, packed, s_w, zp, bias=bias)
    torch.cuda.synchronize()
    L = w4.load_library()
    ws_bytes = w4.w4_linear_workspace_bytes(1, N, K, 8)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    y2 = torch.empty_like(y_eager)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        st = torch.cuda.current_stream().cuda_stream
        w4._check(L.w4_linear(X.data_ptr(), w4.W4_BF16, 1, K, 256, 8, packed.data_ptr(), s_w.data_ptr(),
                              zp.data_ptr() if zp is not None else None, bias.data_ptr(), w4.W4_BF16, None, N,
                              y2.data_ptr(), w4.W4_OUT_BF16, ws.data_ptr(), ws.numel(), st))
    for rep in range(3):
        y2.fill_(0)
        _ = w4.w4_linear(X, 256, 8, packed, s_w, zp, bias=bias)  # eager work between
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y_eager.view(torch.int16)), rep
