"""Mixed-precision decomposition (LLM.int8(): outlier columns in fp16, the rest
W8A8) against the oracle.

- The outlier set (integer work): identical to the oracle's, with the
  position map consistent with it.  Each case first checks on the oracle's
  side that no column's largest |y| lies within 1e-4 of alpha, so the set
  is not decided by fp32 reduction order.
- Codes and scales of the INT8 part: the activation-code and scale rules.
- The outlier values XO: within one fp16 step of fp16(oracle y).
- fp16 outputs: the output tolerance, both for the GEMM fed the oracle's own
  codes / scales / outlier values and for the whole layer.
- The fp16 weight copy: bit-exact.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

from oracle import ref
from tests._match import assert_codes, assert_scales, assert_y, say
from zq_workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALPHA = 6.0


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


def workload(M, K, N, G, dt, pre, act, bias, frac, gain, seed=0, logscale=0.0):
    return Workload("decomp_case", M, K, N, G, dt, pre, act, bias, logscale, 0.02, 0.0, frac, gain,
                    False, seed=seed)


def check_not_borderline(Y, alpha):
    colmax = np.max(np.abs(Y.astype(np.float64)), axis=0)
    near = np.abs(colmax - alpha) <= 1e-4 * max(abs(alpha), 1.0)
    assert not near.any(), f"columns {np.nonzero(near)[0]} sit on the threshold"


def check_set(slot, cols, want):
    P = int(cols[0])
    assert P == want.size, (P, want.size)
    assert np.array_equal(cols[1:1 + P], want)
    expect = np.full(slot.shape, -1, dtype=np.int64)
    expect[want] = np.arange(want.size)
    assert np.array_equal(slot.astype(np.int64), expect)


# (M, K, pre, x dtype, outlier fraction, gain, seed)
PROLOGUE_CASES = [
    (64, 1024, ref.PRE_LAYERNORM, "f16", 0.01, 60.0, 1),
    (300, 768, ref.PRE_LAYERNORM, "f32", 0.005, 100.0, 2),     # ragged token count
    (7, 10240, ref.PRE_LAYERNORM, "f16", 0.002, 100.0, 3),     # 16 waves per token
    (33, 512, ref.PRE_GELU, "f16", 0.02, 10.0, 4),
    (20, 256, ref.PRE_NONE, "f32", 0.03, 8.0, 5),
    (16, 28672, ref.PRE_GELU, "f16", 0.001, 10.0, 6),          # the decode row length
    (129, 2048, ref.PRE_LAYERNORM, "f16", 0.0, 1.0, 7),        # no outlier channel
    # few tokens with long rows: marks by column segment, INT8 part by row segment
    (40, 10000, ref.PRE_NONE, "f32", 0.01, 20.0, 9),           # ragged segments, M > 16
    (64, 4096, ref.PRE_GELU, "f32", 0.005, 10.0, 10),          # largest M, shortest K there
    (5, 6160, ref.PRE_LAYERNORM, "f32", 0.01, 80.0, 11),
    (1, 8192, ref.PRE_NONE, "f16", 0.002, 30.0, 12),
]


@pytest.mark.parametrize("M,K,pre,dt,frac,gain,seed", PROLOGUE_CASES)
def test_outlier_set_and_prologue(zq, M, K, pre, dt, frac, gain, seed):
    say("decomp prologue", M, K, pre, dt, frac, gain, seed)
    w = workload(M, K, 64, 64, dt, pre, 0, False, frac, gain, seed)
    X = make_inputs(w).X
    Y = ref.preop(X, pre)
    check_not_borderline(Y, ALPHA)
    want = ref.outlier_columns(Y, ALPHA)
    if frac > 0:
        assert want.size > 0
    q_ref, s_ref = ref.quantize_rows_excluding(Y, want)

    Xd = dev(X)
    slot, cols = zq.outlier_columns(Xd, ALPHA, pre)
    check_set(host(slot), host(cols), want)
    Xq, s_x, XO = zq.ln_quant_decomp(Xd, slot, pre)
    assert_codes(host(Xq), q_ref)
    assert_scales(host(s_x), s_ref)
    xo = host(XO)[:, :want.size].astype(np.float64)
    xo_ref = ref.round_to_f16(Y[:, want]).astype(np.float16)
    step = np.spacing(np.abs(xo_ref)).astype(np.float64)
    assert np.all(np.abs(xo - xo_ref.astype(np.float64)) <= step)


@pytest.mark.parametrize("alpha,every", [(-1.0, True), (1e30, False), (float("nan"), False)])
def test_outlier_set_extremes(zq, alpha, every):
    say("decomp extremes", alpha)
    w = workload(40, 256, 64, 64, "f16", ref.PRE_LAYERNORM, 0, False, 0.02, 50.0, 8)
    X = make_inputs(w).X
    want = np.arange(256) if every else np.zeros(0, dtype=np.int64)
    assert np.array_equal(ref.outlier_columns(ref.preop(X, ref.PRE_LAYERNORM), alpha), want)
    slot, cols = zq.outlier_columns(dev(X), alpha, ref.PRE_LAYERNORM)
    check_set(host(slot), host(cols), want)


@pytest.mark.parametrize("pre", [ref.PRE_GELU, ref.PRE_NONE])
@pytest.mark.parametrize("alpha,every", [(-1.0, True), (float("nan"), False)])
def test_few_token_extremes(zq, pre, alpha, every):
    """Few tokens with long rows: every column an outlier (nothing left for the
    INT8 part: scale 0, codes 0) and none (the plain prologue's codes)."""
    say("decomp few-token extremes", pre, alpha)
    w = workload(16, 8192, 64, 64, "f16", pre, 0, False, 0.002, 10.0, 13)
    X = make_inputs(w).X
    Y = ref.preop(X, pre)
    want = ref.outlier_columns(Y, alpha)
    assert want.size == (8192 if every else 0)
    Xd = dev(X)
    slot, cols = zq.outlier_columns(Xd, alpha, pre)
    check_set(host(slot), host(cols), want)
    Xq, s_x, XO = zq.ln_quant_decomp(Xd, slot, pre)
    q_ref, s_ref = ref.quantize_rows_excluding(Y, want)
    assert_codes(host(Xq), q_ref)
    assert_scales(host(s_x), s_ref)
    if every:
        assert not host(Xq).any() and not host(s_x).any()


def test_few_token_gelu_negative_side(zq):
    """GeLU rows whose columns outside O are all at most 0.3, so the INT8 part's
    scale comes from the negative side (the L and R of the rule), while the
    outlier columns hold large positive values."""
    say("decomp few-token gelu negative side")
    rng = np.random.default_rng(14)
    M, K = 16, 8192
    X = -np.abs(rng.standard_normal((M, K))).astype(np.float32) * 2.0
    X[:, rng.choice(K, 12, replace=False)] = 10.0 + rng.random((M, 12)).astype(np.float32)
    X = X.astype(np.float16)
    Y = ref.preop(X, ref.PRE_GELU)
    check_not_borderline(Y, ALPHA)
    want = ref.outlier_columns(Y, ALPHA)
    assert want.size == 12
    Xd = dev(X)
    slot, cols = zq.outlier_columns(Xd, ALPHA, ref.PRE_GELU)
    check_set(host(slot), host(cols), want)
    Xq, s_x, XO = zq.ln_quant_decomp(Xd, slot, ref.PRE_GELU)
    q_ref, s_ref = ref.quantize_rows_excluding(Y, want)
    assert_codes(host(Xq), q_ref)
    assert_scales(host(s_x), s_ref)
    assert np.all(host(s_x) < 0.2 / 127 + 1e-6)    # the negative side decided every scale


@pytest.mark.parametrize("N,K,dt", [(200, 96, np.float32), (64, 5120, np.float16),
                                    (13, 16, np.float32)])
def test_pack_outlier_weights_exact(zq, N, K, dt):
    say("decomp weights", N, K, dt.__name__)
    rng = np.random.default_rng(N * K)
    W = (0.05 * rng.standard_normal((N, K))).astype(dt)
    W[0, 0] = 70000.0 if dt == np.float32 else 1.0       # rounds to +inf in fp16
    want = ref.round_to_f16(W.astype(np.float32)).astype(np.float16).T
    got = host(zq.pack_outlier_weights(dev(W)))
    assert np.array_equal(got.view(np.uint16), np.ascontiguousarray(want).view(np.uint16))


def _oracle_operands(X, W, pre, G, alpha):
    Y = ref.preop(X, pre)
    cols = ref.outlier_columns(Y, alpha)
    Xq, s_x = ref.quantize_rows_excluding(Y, cols)
    Wq, s_w = ref.quantize_groups(W, G)
    return Y, cols, Xq, s_x, Wq, s_w


# (M, N, K, G, act, bias, outlier fraction, gain, alpha, seed)
GEMM_CASES = [
    (300, 388, 512, 4, ref.ACT_NONE, True, 0.03, 40.0, ALPHA, 11),      # ragged, P ~ 15
    (256, 384, 768, 128, ref.ACT_GELU, True, 0.05, 40.0, ALPHA, 12),    # P ~ 38: 3 chunks
    (77, 1000, 256, 1, ref.ACT_NONE, False, 0.0, 1.0, ALPHA, 13),       # P = 0
    (96, 128, 256, 1, ref.ACT_GELU, True, 0.02, 40.0, -1.0, 14),        # P = K
    (1024, 1536, 1024, 1, ref.ACT_NONE, True, 0.01, 60.0, ALPHA, 15),   # the large tiles
    # 256x192 tiles with P = 20 (operands staged in LDS) and a ragged last N tile
    (4096, 2848, 256, 1, ref.ACT_GELU, True, 0.08, 40.0, ALPHA, 16),
    # few tokens: the weight-streaming kernel, ragged last workgroup, P ~ 20
    (16, 1000, 2048, 1, ref.ACT_NONE, True, 0.01, 60.0, ALPHA, 17),
    # M = 32 with more than 64 outlier columns (list read from global memory)
    (32, 512, 4096, 8, ref.ACT_GELU, True, 0.02, 60.0, ALPHA, 18),
    # few tokens, P <= 32: operands staged in LDS for 32 tokens; N % 8 == 4 reads them directly
    (32, 1024, 2048, 1, ref.ACT_GELU, True, 0.008, 60.0, ALPHA, 19),
    (9, 1004, 1024, 4, ref.ACT_NONE, True, 0.01, 60.0, ALPHA, 20),
]


@pytest.mark.parametrize("M,N,K,G,act,bias,frac,gain,alpha,seed", GEMM_CASES)
def test_gemm_decomp_on_oracle_operands(zq, M, N, K, G, act, bias, frac, gain, alpha, seed):
    say("decomp gemm", M, N, K, G, act, bias, frac, alpha, seed)
    inp = make_inputs(workload(M, K, N, G, "f16", ref.PRE_LAYERNORM, act, bias, frac, gain, seed))
    Y, cols, Xq, s_x, Wq, s_w = _oracle_operands(inp.X, inp.W, ref.PRE_LAYERNORM, G, alpha)
    if frac > 0 or alpha < 0:
        assert cols.size > 0
    acc = ref.gemm_i32(Xq, Wq)
    want = ref.decomp_epilogue(acc, s_x, s_w, G, Y, cols, inp.W, inp.bias, act)

    XO = np.zeros((M, K), dtype=np.float16)
    XO[:, :cols.size] = ref.round_to_f16(Y[:, cols]).astype(np.float16)
    cl = np.zeros(K + 1, dtype=np.int32)
    cl[0] = cols.size
    cl[1:1 + cols.size] = cols
    Wt = np.ascontiguousarray(ref.round_to_f16(inp.W).astype(np.float16).T)
    got = zq.w8a8_gemm_decomp(dev(Xq), dev(s_x), dev(Wq), dev(s_w), G, dev(cl), dev(XO), dev(Wt),
                              None if inp.bias is None else dev(inp.bias), act)
    assert_y(host(got), want)


# Shapes whose 256 x 192 tiles would leave a last round at most half full, so
# the columns past the last whole round go to a second launch of 128 x 192
# tiles: a 4-column tail whose output rows (N % 8 == 4) rule out the LDS
# panels, and a 1024-column tail whose interior tiles take them (P <= 32).
# Sampled tokens, every column.
@pytest.mark.parametrize("M,N,K,G,act,frac,seed", [
    (1796, 18436, 256, 4, ref.ACT_GELU, 0.03, 31),
    (4096, 13312, 256, 128, ref.ACT_NONE, 0.04, 32),
])
def test_gemm_decomp_round_split(zq, M, N, K, G, act, frac, seed):
    say("decomp gemm round split", M, N, K, G, act, frac, seed)
    inp = make_inputs(workload(M, K, N, G, "f16", ref.PRE_LAYERNORM, act, True, frac, 40.0, seed))
    Y, cols, Xq, s_x, Wq, s_w = _oracle_operands(inp.X, inp.W, ref.PRE_LAYERNORM, G, ALPHA)
    assert 0 < cols.size <= 32
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), rng.integers(0, M, 32)]))
    acc = ref.gemm_i32(Xq[rows], Wq)
    want = ref.decomp_epilogue(acc, s_x[rows], s_w, G, Y[rows], cols, inp.W, inp.bias, act)
    XO = np.zeros((M, K), dtype=np.float16)
    XO[:, :cols.size] = ref.round_to_f16(Y[:, cols]).astype(np.float16)
    cl = np.zeros(K + 1, dtype=np.int32)
    cl[0] = cols.size
    cl[1:1 + cols.size] = cols
    Wt = np.ascontiguousarray(ref.round_to_f16(inp.W).astype(np.float16).T)
    got = zq.w8a8_gemm_decomp(dev(Xq), dev(s_x), dev(Wq), dev(s_w), G, dev(cl), dev(XO), dev(Wt),
                              dev(inp.bias), act)
    assert_y(host(got)[rows], want)


# (M, N, K, G, pre, act, x dtype, bias, outlier fraction, gain, seed)
LAYER_CASES = [
    (200, 256, 1024, 1, ref.PRE_LAYERNORM, ref.ACT_NONE, "f16", True, 0.01, 60.0, 21),
    (131, 392, 768, 8, ref.PRE_LAYERNORM, ref.ACT_GELU, "f32", True, 0.005, 100.0, 22),
    (64, 512, 512, 128, ref.PRE_GELU, ref.ACT_NONE, "f16", False, 0.02, 10.0, 23),
    (16, 1024, 10240, 1, ref.PRE_LAYERNORM, ref.ACT_NONE, "f16", True, 0.002, 100.0, 24),
    (40, 256, 512, 1, ref.PRE_NONE, ref.ACT_GELU, "f32", True, 0.01, 8.0, 25),
]


@pytest.mark.parametrize("M,N,K,G,pre,act,dt,bias,frac,gain,seed", LAYER_CASES)
def test_linear_decomp(zq, M, N, K, G, pre, act, dt, bias, frac, gain, seed):
    say("decomp layer", M, N, K, G, pre, act, dt, frac, seed)
    inp = make_inputs(workload(M, K, N, G, dt, pre, act, bias, frac, gain, seed, logscale=0.3))
    check_not_borderline(ref.preop(inp.X, pre), ALPHA)
    Wq_r, s_w_r = ref.quantize_groups(inp.W, G)
    want, q_ref, s_ref, cols = ref.linear_decomp(inp.X, pre, None, None, 1e-5, ALPHA, Wq_r, s_w_r,
                                                 G, inp.W, inp.bias, act)
    assert cols.size > 0

    Wd = dev(inp.W)
    Wq, s_w = zq.quantize_weights_grouped(Wd, G)
    assert np.array_equal(host(Wq), Wq_r) and np.array_equal(host(s_w), s_w_r)
    Wt = zq.pack_outlier_weights(Wd)
    got = zq.linear_w8a8_decomp(dev(inp.X), Wq, s_w, G, Wt, ALPHA, pre,
                                bias=None if inp.bias is None else dev(inp.bias), act=act)
    assert_y(host(got), want)


def test_linear_decomp_outlier_workload_full_size(zq):
    """The outlier workload (X fp16 [4096 x 5120], N(0,1) with 0.5% of the
    channels x100, LayerNorm; W [13824 x 5120]) with the decomposition in
    place of the SmoothQuant fold and per-output-channel weight scales (G = 1):
    the outlier set in full, codes, scales and outputs on sampled tokens."""
    w = dataclasses.replace(WORKLOADS["outlier_smooth"], group_rows=1, smooth=False)
    say("decomp full size", w.M, w.K, w.N)
    inp = make_inputs(w)
    G = 1
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w.M - 1],
                                     np.linspace(0, w.M - 1, 40).astype(np.int64)]))
    Wq_r, s_w_r = ref.quantize_groups(inp.W, G)
    want, q_ref, s_ref, cols = ref.linear_decomp_rows(inp.X, w.pre, inp.gamma, inp.beta, w.eps,
                                                      ALPHA, Wq_r, s_w_r, G, inp.W, inp.bias,
                                                      w.act, rows)
    assert np.array_equal(cols, inp.outlier_channels)

    Xd = dev(inp.X)
    Wd = dev(inp.W)
    Wq, s_w = zq.quantize_weights_grouped(Wd, G)
    assert np.array_equal(host(Wq), Wq_r) and np.array_equal(host(s_w), s_w_r)
    Wt = zq.pack_outlier_weights(Wd)
    del Wd
    slot, cl = zq.outlier_columns(Xd, ALPHA, w.pre, dev(inp.gamma), dev(inp.beta), w.eps)
    check_set(host(slot), host(cl), cols)
    Xq, s_x, _ = zq.ln_quant_decomp(Xd, slot, w.pre, dev(inp.gamma), dev(inp.beta), w.eps)
    assert_codes(host(Xq)[rows], q_ref)
    assert_scales(host(s_x)[rows], s_ref)
    got = zq.linear_w8a8_decomp(Xd, Wq, s_w, G, Wt, ALPHA, w.pre, dev(inp.gamma), dev(inp.beta),
                                w.eps)
    assert_y(host(got)[rows], want)


def test_linear_decomp_decode_size(zq):
    """The decode shape (X fp16 [16 x 28672] through the GeLU prologue, W
    [8192 x 28672], G = 128) with 0.1% of the channels x10: the
    weight-streaming kernel with the fp16 part, all 16 tokens against the oracle."""
    w = workload(16, 28672, 8192, 128, "f16", ref.PRE_GELU, ref.ACT_NONE, False, 0.001, 10.0, 19)
    say("decomp decode size", w.M, w.K, w.N)
    inp = make_inputs(w)
    check_not_borderline(ref.preop(inp.X, w.pre), ALPHA)
    Wq_r, s_w_r = ref.quantize_groups(inp.W, w.group_rows)
    want, q_ref, s_ref, cols = ref.linear_decomp(inp.X, w.pre, None, None, 1e-5, ALPHA, Wq_r,
                                                 s_w_r, w.group_rows, inp.W, None, w.act)
    assert cols.size > 0
    Wd = dev(inp.W)
    Wq, s_w = zq.quantize_weights_grouped(Wd, w.group_rows)
    assert np.array_equal(host(Wq), Wq_r) and np.array_equal(host(s_w), s_w_r)
    Wt = zq.pack_outlier_weights(Wd)
    del Wd
    got = zq.linear_w8a8_decomp(dev(inp.X), Wq, s_w, w.group_rows, Wt, ALPHA, w.pre)
    assert_y(host(got), want)
