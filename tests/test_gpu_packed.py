"""Packed weights for the weight-streaming GEMM: the re-layout itself, and the
packed GEMM / layer against the oracle and against the row-major calls, which
must agree bit for bit (same codes, same scales, same kernel arithmetic)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from tests._match import assert_y, say
from zq_workloads import WORKLOADS, make_inputs, random_int8

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


def packed_layout(Wq):
    """The layout zq.h defines, written with numpy: zero-pad to 32-row and
    512-byte multiples, then order blocks (row block, k block), rows, bytes."""
    N, K = Wq.shape
    nb, ks = -(-N // 32), -(-K // 512)
    P = np.zeros((nb * 32, ks * 512), dtype=np.int8)
    P[:N, :K] = Wq
    return P.reshape(nb, 32, ks, 512).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("N,K", [(32, 512), (100, 208), (64, 1040), (4, 16), (260, 4096)])
def test_pack_layout(zq, N, K):
    say("pack", N, K)
    rng = np.random.default_rng(N + K)
    Wq = random_int8(rng, (N, K))
    got = host(zq.pack_weights(dev(Wq)))
    assert np.array_equal(got, packed_layout(Wq))


SHAPES = [(1, 32, 512), (5, 100, 208), (16, 256, 512), (17, 64, 1024), (32, 132, 4096),
          (16, 48, 16), (3, 8, 28672), (16, 96, 1040)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_packed_gemm_int32_bit_exact(zq, M, N, K):
    say("packed i32", M, N, K)
    rng = np.random.default_rng(M * 17 + N * 3 + K)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    Wp = zq.pack_weights(dev(Wq))
    got = host(zq.w8a8_gemm_dequant_packed(dev(Xq), None, Wp, None, 4, N, out_dtype=torch.int32))
    assert np.array_equal(got, ref.gemm_i32(Xq, Wq))


@pytest.mark.parametrize("M,N,K,G,act", [(16, 192, 320, 64, 1), (24, 260, 1040, 4, 0),
                                         (1, 64, 512, 64, 1), (32, 512, 2048, 128, 0)])
def test_packed_gemm_f16_equals_row_major(zq, M, N, K, G, act):
    say("packed f16", M, N, K, G, act)
    rng = np.random.default_rng(M + N + K + G)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    s_x = (np.exp(rng.standard_normal(M)) * 0.01).astype(np.float32)
    s_w = (np.exp(rng.standard_normal(N // G)) * 2e-4).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    Wp = zq.pack_weights(dev(Wq))
    guard = 4096
    buf = torch.full((M * N + guard,), 7.0, dtype=torch.float16, device="cuda")
    zq.w8a8_gemm_dequant_packed(dev(Xq), dev(s_x), Wp, dev(s_w), G, N, dev(bias), act,
                                out=buf[:M * N].view(M, N))
    flat = host(buf)
    assert np.all(flat[M * N:] == 7.0)
    got = flat[:M * N].reshape(M, N)
    row = host(zq.w8a8_gemm_dequant(dev(Xq), dev(s_x), dev(Wq), dev(s_w), G, dev(bias), act,
                                    path=zq.PATH_SKINNY))
    assert np.array_equal(got.view(np.uint16), row.view(np.uint16))
    assert_y(got, ref.epilogue(ref.gemm_i32(Xq, Wq), s_x, s_w, G, bias, act))


@pytest.mark.parametrize("name", ["tiny", "decode_ffn_down"])
def test_packed_linear_equals_row_major(zq, name):
    """The whole layer with packed weights gives the row-major layer's output
    bit for bit, at the workload's full size."""
    w = WORKLOADS[name]
    M = min(w.M, 32)
    say("packed linear", name, M)
    inp = make_inputs(w, M=M)
    X = dev(inp.X)
    Wq, s_w = zq.quantize_weights_grouped(dev(inp.W), w.group_rows)
    Wp = zq.pack_weights(Wq)
    bias = dev(inp.bias) if inp.bias is not None else None
    kw = dict(pre=w.pre, gamma=dev(inp.gamma), beta=dev(inp.beta), eps=w.eps, bias=bias,
              act=w.act)
    Y_row = host(zq.linear_w8a8(X, Wq, s_w, w.group_rows, **kw))
    Y_pack = host(zq.linear_w8a8_packed(X, Wp, s_w, w.group_rows, w.N, **kw))
    assert np.array_equal(Y_row.view(np.uint16), Y_pack.view(np.uint16))
