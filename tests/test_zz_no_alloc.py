"""zq_linear_w8a8_noalloc (for callers that cannot allocate) against
zq_linear_w8a8 through the C ABI: bit-identical outputs on two calls in a
row, the second with a smaller input; sizes beyond the fixed array are
rejected before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest

from tests._match import say
from zq_workloads import random_affine, random_int8

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def zq():
    import post_w8a8_quantized_amd as m
    assert torch.cuda.is_available(), "a GPU device node exists but torch sees no GPU"
    m.library()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _case(rng, M, K, N, G, dt):
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(dt)
    g, b = random_affine(rng, K)
    Wq = random_int8(rng, (N, K))
    s_w = (np.exp(rng.standard_normal(N // G)) * 2e-4).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    return [dev(v) for v in (X, Wq, s_w, g, b, bias)]


@pytest.mark.parametrize("first,second", [
    ((1024, 2048, 768, 128, np.float16, 1, 0), (200, 512, 384, 64, np.float32, 0, 1)),
    ((4096, 5120, 512, 128, np.float16, 1, 0), (16, 4096, 256, 128, np.float16, 2, 1)),
])
def test_noalloc_matches_linear_twice(zq, first, second):
    """Two calls in a row on the shared array, the second smaller (and through
    the few-token path in the second case): each equals zq_linear_w8a8 on a
    workspace of its own, bit for bit."""
    rng = np.random.default_rng(sum(first[:3]) + sum(second[:3]))
    for (M, K, N, G, dt, pre, act) in (first, second):
        say("noalloc", M, K, N, G, dt.__name__, pre, act)
        X, Wq, s_w, g, b, bias = _case(rng, M, K, N, G, dt)
        gg, bb = (g, b) if pre == zq.PRE_LAYERNORM else (None, None)
        want = host(zq.linear_w8a8(X, Wq, s_w, G, pre, gg, bb, 1e-5, bias, act))
        Y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
        zq.linear_w8a8_noalloc(X, Wq, s_w, G, pre, gg, bb, 1e-5, bias, act, out=Y)
        got = host(Y)
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_noalloc_rejects_sizes_beyond_the_array(zq):
    """zq_linear_workspace_bytes(M, K) above ZQ_NOALLOC_SCRATCH_BYTES returns
    ZQ_ERR_WORKSPACE and leaves the output untouched."""
    say("noalloc too large")
    M, K, N, G = 8200, 4096, 64, 64
    assert zq.linear_workspace_bytes(M, K) > zq.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Wq = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    s_w = torch.ones(N // G, dtype=torch.float32, device="cuda")
    Y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(zq.ZQError, match="ZQ_ERR_WORKSPACE"):
        zq.linear_w8a8_noalloc(X, Wq, s_w, G, out=Y)
    assert bool((Y == 7.0).all())


def test_noalloc_captured_in_a_graph(zq):
    """The callers it is for: captured in a HIP graph, every replay gives the
    eager zq_linear_w8a8 bits, with an eager no-alloc call on other inputs (which
    overwrites the shared array) and unrelated work between the replays."""
    say("noalloc graph")
    rng = np.random.default_rng(9)
    M, K, N, G = 300, 768, 512, 128
    X, Wq, s_w, g, b, bias = _case(rng, M, K, N, G, np.float16)
    X2 = dev((rng.standard_normal((M, K)) * 3).astype(np.float16))
    want = host(zq.linear_w8a8(X, Wq, s_w, G, zq.PRE_LAYERNORM, g, b, 1e-5, bias, zq.ACT_GELU))
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    Y2 = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def call():
        zq.linear_w8a8_noalloc(X, Wq, s_w, G, zq.PRE_LAYERNORM, g, b, 1e-5, bias, zq.ACT_GELU,
                               out=Y)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        Y.fill_(0)
        zq.linear_w8a8_noalloc(X2, Wq, s_w, G, out=Y2)       # overwrites the array
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint16), want.view(np.uint16)), f"replay {r}"
        del junk
