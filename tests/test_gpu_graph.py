"""The layer captured in a HIP graph (as the benchmark runs it) gives, on every
replay, the same bits as the eager call, with unrelated eager work and
synchronisations between the replays.  The same holds for the FFN block, the
FP8 layer and the decomposed layer, which the benchmark also replays."""
from __future__ import annotations

import numpy as np
import pytest

from tests._match import say
from zq_workloads import random_affine, random_int8

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


# (M, K, N, G): the weight-streaming and the tiled GEMM, and a shape whose GEMM
# is the round split (two launches: 256x256 tiles, then 128x192 tiles)
@pytest.mark.parametrize("M,K,N,G", [(16, 768, 512, 128), (300, 768, 512, 128),
                                     (1796, 256, 18436, 4)])
def test_graph_replays_match_eager(M, K, N, G):
    import post_w8a8_quantized_amd as zq
    say("graph replay", M, K, N, G)
    rng = np.random.default_rng(M)
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)).cuda()
    g, b = (torch.from_numpy(a).cuda() for a in random_affine(rng, K))
    Wq = torch.from_numpy(random_int8(rng, (N, K))).cuda()
    s_w = torch.from_numpy(np.full(N // G, 2e-3, np.float32)).cuda()
    bias = torch.from_numpy((0.01 * rng.standard_normal(N)).astype(np.float32)).cuda()
    ws = torch.empty(zq.linear_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def call():
        zq.linear_w8a8(X, Wq, s_w, G, zq.PRE_LAYERNORM, g, b, 1e-5, bias, zq.ACT_GELU,
                       workspace=ws, out=Y)

    call()
    torch.cuda.synchronize()
    eager = Y.cpu().numpy().view(np.uint16).copy()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(4):
        Y.fill_(0)
        ws.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = Y.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, eager), f"replay {r} differs"
        del junk


@pytest.mark.parametrize("M", [16, 300])
def test_graph_replays_match_eager_decomposition(M):
    """The decomposed layer (outlier search, prologue, GEMM with the fp16 part)
    under capture: its workspace starts from different garbage on every replay
    (the search clears its own marks with a kernel, not a memset)."""
    import post_w8a8_quantized_amd as zq
    say("graph replay decomposition", M)
    rng = np.random.default_rng(M + 1)
    K, N, G = 768, 512, 1
    Xh = rng.standard_normal((M, K)).astype(np.float32)
    Xh[:, [5, 300, 301, 700]] *= 40.0
    X = torch.from_numpy(Xh.astype(np.float16)).cuda()
    W = torch.from_numpy((0.02 * rng.standard_normal((N, K))).astype(np.float32)).cuda()
    Wq, s_w = zq.quantize_weights_grouped(W, G)
    Wt = zq.pack_outlier_weights(W)
    bias = torch.from_numpy((0.01 * rng.standard_normal(N)).astype(np.float32)).cuda()
    ws = torch.empty(zq.linear_decomp_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def call():
        zq.linear_w8a8_decomp(X, Wq, s_w, G, Wt, 6.0, zq.PRE_LAYERNORM, None, None, 1e-5, bias,
                              zq.ACT_GELU, workspace=ws, out=Y)

    call()
    torch.cuda.synchronize()
    eager = Y.cpu().numpy().view(np.uint16).copy()
    P = int(ws[(K * 4 + 255) // 256 * 256:][:4].view(torch.int32).item())
    assert P >= 4

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(4):
        Y.fill_(0)
        ws.fill_(255 if r % 2 else 1)
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = Y.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, eager), f"replay {r} differs"
        del junk


def _check_replays(call, Y, ws, fills=(0, 0, 0, 0)):
    """Eager result, then a captured graph replayed len(fills) times; before each
    replay Y is cleared and the workspace filled with the given byte."""
    call()
    torch.cuda.synchronize()
    eager = Y.cpu().numpy().view(np.uint16).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r, v in enumerate(fills):
        Y.fill_(0)
        ws.fill_(v)
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = Y.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, eager), f"replay {r} differs"
        del junk


@pytest.mark.parametrize("M", [16, 300])
def test_graph_replays_match_eager_ffn(M):
    """The chained FFN block: its FFN-up epilogue writes every partial row
    maximum that H's quantizer reads (plain stores), so garbage left in the
    workspace between replays changes nothing."""
    import post_w8a8_quantized_amd as zq
    say("graph replay ffn", M)
    rng = np.random.default_rng(M + 2)
    K, F, G = 256, 1024, 128
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)).cuda()
    g, b = (torch.from_numpy(a).cuda() for a in random_affine(rng, K))
    W1q = torch.from_numpy(random_int8(rng, (F, K))).cuda()
    W2q = torch.from_numpy(random_int8(rng, (K, F))).cuda()
    s1 = torch.from_numpy(np.full(F // G, 2e-3, np.float32)).cuda()
    s2 = torch.from_numpy(np.full(K // G, 1e-3, np.float32)).cuda()
    b1 = torch.from_numpy((0.01 * rng.standard_normal(F)).astype(np.float32)).cuda()
    b2 = torch.from_numpy((0.01 * rng.standard_normal(K)).astype(np.float32)).cuda()
    ws = torch.empty(zq.ffn_workspace_bytes(M, K, F), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, K), dtype=torch.float16, device="cuda")

    def call():
        zq.ffn_w8a8(X, W1q, s1, G, W2q, s2, G, g, b, 1e-5, b1, b2, workspace=ws, out=Y)

    _check_replays(call, Y, ws, fills=(0, 255, 0x7f, 1))


@pytest.mark.parametrize("M", [16, 300])
def test_graph_replays_match_eager_fp8(M):
    import post_w8a8_quantized_amd as zq
    say("graph replay fp8", M)
    rng = np.random.default_rng(M + 3)
    K, N, G = 768, 512, 128
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)).cuda()
    g, b = (torch.from_numpy(a).cuda() for a in random_affine(rng, K))
    W = torch.from_numpy((0.02 * rng.standard_normal((N, K))).astype(np.float32)).cuda()
    Wq8, s_w = zq.quantize_weights_grouped_fp8(W, G)
    bias = torch.from_numpy((0.01 * rng.standard_normal(N)).astype(np.float32)).cuda()
    ws = torch.empty(zq.linear_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def call():
        zq.linear_w8a8_fp8(X, Wq8, s_w, G, zq.PRE_LAYERNORM, g, b, 1e-5, bias, zq.ACT_GELU,
                           workspace=ws, out=Y)

    _check_replays(call, Y, ws, fills=(0, 255, 0, 1))
