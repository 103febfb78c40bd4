"""The unfused order (op -> fp16 tensor -> quantizer -> int32 GEMM -> dequantizer),
kept to measure the fusion gain: its intermediates against the oracle's unfused
prologue, and its output bit-identical to the fused GEMM epilogue on the same
codes."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from tests._match import assert_codes, assert_scales, assert_y, say
from zq_workloads import WORKLOADS, make_inputs, random_affine, random_int8

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


def r256(v):
    return (v + 255) // 256 * 256


def split_ws(ws, M, N, K):
    w = host(ws)
    o1 = r256(2 * M * K)
    o2 = o1 + r256(M * K)
    o3 = o2 + r256(4 * M)
    y16 = w[:2 * M * K].view(np.float16).reshape(M, K)
    q = w[o1:o1 + M * K].view(np.int8).reshape(M, K)
    s = w[o2:o2 + 4 * M].view(np.float32)
    acc = w[o3:o3 + 4 * M * N].view(np.int32).reshape(M, N)
    return y16, q, s, acc


@pytest.mark.parametrize("M,K,N,pre,dt,act,affine", [
    (16, 256, 256, ref.PRE_LAYERNORM, np.float32, 0, True),
    (200, 768, 384, ref.PRE_LAYERNORM, np.float16, 1, False),
    (37, 4096, 132, ref.PRE_GELU, np.float16, 0, False),
    (5, 10240, 64, ref.PRE_LAYERNORM, np.float16, 1, True),   # 16 waves per token
    (16, 28672, 256, ref.PRE_GELU, np.float16, 0, False),
    (33, 1040, 96, ref.PRE_NONE, np.float16, 1, False),
])
def test_unfused_layer(zq, M, K, N, pre, dt, act, affine):
    say("unfused", M, K, N, pre, dt.__name__, act)
    rng = np.random.default_rng(M + K + N)
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(dt)
    g, b = random_affine(rng, K) if affine else (None, None)
    G = 4
    Wq = random_int8(rng, (N, K))
    s_w = (np.exp(rng.standard_normal(N // G)) * 2e-4).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    ws = torch.zeros(zq.linear_unfused_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    gd = None if g is None else dev(g)
    bd = None if b is None else dev(b)
    Y = host(zq.linear_w8a8_unfused(dev(X), dev(Wq), dev(s_w), G, pre, gd, bd, 1e-5, dev(bias),
                                    act, workspace=ws))
    y16, q, s, acc = split_ws(ws, M, N, K)

    # (1) the op's fp16 tensor: the oracle's op rounded to fp16.  The two sides'
    # fp32 values differ by rounding order only: the GPU's y carries a few fp32
    # roundings of its own inputs (x - mean, rstd * gamma, + beta), so its error
    # is a few ulps of the element plus a few ulps of the row's largest |y| (an
    # element near 0 after cancellation).  An element may therefore round to the
    # other fp16 neighbour only where the oracle's value sits that close to the
    # midpoint between the two (a near-tie: both roundings are correct).
    y32 = ref.preop(X, pre, g, b, 1e-5)
    y_ref = ref.round_to_f16(y32).astype(np.float16)
    a, r = y16.astype(np.float64), y_ref.astype(np.float64)
    off = a != r
    if off.any():
        step = np.maximum(np.spacing(np.abs(y16[off])), np.spacing(np.abs(y_ref[off])))
        assert np.all(np.abs(a[off] - r[off]) <= step.astype(np.float64))
        mid = (a[off] + r[off]) / 2
        dist = np.abs(y32[off].astype(np.float64) - mid)
        rowmax = np.broadcast_to(np.abs(y32).max(axis=1, keepdims=True), y32.shape)[off]
        near = 8 * np.spacing(np.abs(y32[off])).astype(np.float64) + 2.0 ** -21 * rowmax
        say(f"unfused fp16 tensor: {int(off.sum())} near-tie roundings of {off.size}, "
            f"largest distance {np.max(dist / near):.3f} of the allowance")
        assert np.all(dist <= near)
    # (2) the quantizer on that tensor: the oracle's quantizer fed the GPU's own
    # fp16 tensor gives the same codes and scales bit for bit; where the two
    # tensors agree the whole unfused prologue agrees exactly
    q_own, s_own = ref.quantize_rows(y16.astype(np.float32))
    assert_codes(q, q_own, exact=True)
    assert np.array_equal(s, s_own)
    q_ref, s_ref = ref.unfused_prologue(X, pre, g, b, 1e-5)
    same = ~off.any(axis=1)
    assert_codes(q[same], q_ref[same], exact=True)
    assert np.array_equal(s[same], s_ref[same])
    # (3) exact accumulators of the GPU's own codes
    assert np.array_equal(acc, ref.gemm_i32(q, Wq))
    # (4) the dequantized output: the fused epilogue's bits for the same codes ...
    Yf = host(zq.w8a8_gemm_dequant(dev(q), dev(s), dev(Wq), dev(s_w), G, dev(bias), act))
    assert np.array_equal(Y.view(np.uint16), Yf.view(np.uint16))
    # ... and the oracle's unfused layer within the output tolerance
    assert_y(Y, ref.epilogue(ref.gemm_i32(q_ref, Wq), s_ref, s_w, G, bias, act))


def test_unfused_bert_workload_sampled(zq):
    """At the BERT FFN-up size: the unfused layer against the oracle's unfused
    order on sampled tokens, with the library's own offline weights."""
    w = WORKLOADS["bert_ffn_up"]
    say("unfused bert")
    inp = make_inputs(w)
    Wq, s_w = zq.quantize_weights_grouped(dev(inp.W), w.group_rows)
    Y = host(zq.linear_w8a8_unfused(dev(inp.X), Wq, s_w, w.group_rows, w.pre, dev(inp.gamma),
                                    dev(inp.beta), w.eps, dev(inp.bias), w.act))
    rows = np.unique(np.concatenate([np.arange(0, w.M, 97), [w.M - 1]]))
    Xs = inp.X[rows]
    q_ref, s_ref = ref.unfused_prologue(Xs, w.pre, inp.gamma, inp.beta, w.eps)
    Wq_h, sw_h = host(Wq), host(s_w)
    Y_ref = ref.epilogue(ref.gemm_i32(q_ref, Wq_h), s_ref, sw_h, w.group_rows, inp.bias, w.act)
    assert_y(Y[rows], Y_ref)
