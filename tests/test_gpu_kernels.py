"""Parity of each HIP entry point with the CPU oracle, through the C ABI.

Sizes span several tiles and ragged tails of the tiled GEMM (each of its tile
shapes: 256 x 256, 256 x 192, 128 x 128 and 128 x 96, with 64- or 128-byte k
slabs) and of the skinny GEMM (16-row blocks, 64-byte k blocks split over 8
waves), plus the degenerate cases of the method.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from tests._match import assert_codes, assert_scales, assert_y, say
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


# ---------------------------------------------------------------- int GEMM

TILED_SHAPES = [
    # M, N, K
    (128, 128, 64),
    (256, 384, 512),
    (130, 260, 208),     # ragged M, N and K tails
    (33, 132, 48),       # one partial tile, K < one slab
    (1000, 516, 784),
    (4096, 256, 128),
    (4096, 8180, 64),    # 256x256 tiles with 4x2 waves, ragged last column tile
    (700, 300, 336),     # 128x96 tiles, ragged M, N and K
]


@pytest.mark.parametrize("M,N,K", TILED_SHAPES)
def test_gemm_tiled_int32_bit_exact(zq, M, N, K):
    say("tiled i32", M, N, K)
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    want = ref.gemm_i32(Xq, Wq)
    got = host(zq.w8a8_gemm_dequant(dev(Xq), None, dev(Wq), None, 4, out_dtype=torch.int32,
                                    path=zq.PATH_TILED))
    assert np.array_equal(got, want)


SKINNY_SHAPES = [
    (1, 16, 64), (5, 100, 208), (16, 256, 512), (17, 64, 1024), (32, 132, 4096),
    (16, 48, 16), (3, 8, 28672),
]


@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_gemm_skinny_int32_bit_exact(zq, M, N, K):
    say("skinny i32", M, N, K)
    rng = np.random.default_rng(M * 11 + N * 5 + K)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    want = ref.gemm_i32(Xq, Wq)
    got = host(zq.w8a8_gemm_dequant(dev(Xq), None, dev(Wq), None, 4, out_dtype=torch.int32,
                                    path=zq.PATH_SKINNY))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("path", ["tiled", "skinny"])
def test_gemm_int32_extremes_at_max_k(zq, path):
    """All codes +-127 at K = 131072: |acc| = 16129 K = 2114060288 < 2^31."""
    say("i32 extremes", path)
    K = 131072
    Xq = np.full((2, K), 127, dtype=np.int8)
    Xq[1] = -127
    Wq = np.full((4, K), 127, dtype=np.int8)
    Wq[2] = -127
    want = ref.gemm_i32(Xq, Wq)
    assert abs(int(want[0, 0])) == 16129 * K
    p = zq.PATH_TILED if path == "tiled" else zq.PATH_SKINNY
    got = host(zq.w8a8_gemm_dequant(dev(Xq), None, dev(Wq), None, 4, out_dtype=torch.int32, path=p))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- epilogue

@pytest.mark.parametrize("path", ["tiled", "skinny"])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("G", [1, 4, 64])
def test_gemm_dequant_epilogue(zq, path, act, G):
    """Same int8 inputs and scales on both sides: only the fp32 (GPU) versus
    fp64 (oracle) epilogue differs, so the result must also sit within one
    fp16 ulp almost everywhere."""
    M = 24 if path == "skinny" else 200
    N, K = 192, 320
    say("epilogue", path, act, G)
    rng = np.random.default_rng(100 + G + act)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    s_x = (np.exp(rng.standard_normal(M)) * 0.01).astype(np.float32)
    s_w = (np.exp(rng.standard_normal(N // G)) * 2e-4).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    want = ref.epilogue(ref.gemm_i32(Xq, Wq), s_x, s_w, G, bias, act)
    p = zq.PATH_TILED if path == "tiled" else zq.PATH_SKINNY
    got = host(zq.w8a8_gemm_dequant(dev(Xq), dev(s_x), dev(Wq), dev(s_w), G, dev(bias), act, path=p))
    assert_y(got, want)
    ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
    off = np.abs(got.astype(np.float64) - want.astype(np.float64)) > ulp
    assert off.mean() <= 1e-3, off.mean()


@pytest.mark.parametrize("path", ["tiled", "skinny"])
def test_gemm_gelu_epilogue_far_range(zq, path):
    """GeLU epilogue over pre-activations far outside the polynomial's fitted
    range [-6.5, 6.5] (the bias carries them out to +-3e4): every output is
    finite and within one fp16 ulp of fp16(exact GeLU), so GeLU(v) = v for
    large v and -0 or 0 for large negative v."""
    M = 24 if path == "skinny" else 200
    N, K, G = 192, 64, 4
    say("gelu far range", path)
    rng = np.random.default_rng(7)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    s_x = (np.exp(rng.standard_normal(M)) * 1e-3).astype(np.float32)
    s_w = (np.exp(rng.standard_normal(N // G)) * 1e-4).astype(np.float32)
    mag = 10.0 ** rng.uniform(-2.0, np.log10(3e4), N)
    bias = (np.where(np.arange(N) % 2 == 0, 1.0, -1.0) * mag).astype(np.float32)
    want = ref.epilogue(ref.gemm_i32(Xq, Wq), s_x, s_w, G, bias, ref.ACT_GELU)
    p = zq.PATH_TILED if path == "tiled" else zq.PATH_SKINNY
    got = host(zq.w8a8_gemm_dequant(dev(Xq), dev(s_x), dev(Wq), dev(s_w), G, dev(bias),
                                    zq.ACT_GELU, path=p))
    assert np.all(np.isfinite(got))
    w64 = want.astype(np.float64)
    ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - w64) <= ulp)
    big = np.abs(w64) >= 8.0
    assert big.sum() > M * N // 6
    assert np.array_equal(got[big], want[big])


@pytest.mark.parametrize("M,N,K", TILED_SHAPES + [(520, 392, 256), (300, 204, 96)])
def test_gemm_tiled_f16_tile_edges(zq, M, N, K):
    """fp16 output of the tiled kernel at tile multiples and at ragged M and N
    tails, including rows of Y that are only 8-byte aligned (N % 8 == 4)."""
    say("tiled f16 edges", M, N, K)
    rng = np.random.default_rng(M * 13 + N * 7 + K)
    G = 4
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    s_x = (np.exp(rng.standard_normal(M)) * 0.01).astype(np.float32)
    s_w = (np.exp(rng.standard_normal(N // G)) * 2e-4).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    act = (M + N) % 2
    want = ref.epilogue(ref.gemm_i32(Xq, Wq), s_x, s_w, G, bias, act)
    # Y sits at the start of a larger buffer whose tail must stay untouched.
    guard = 4096
    buf = torch.full((M * N + guard,), 7.0, dtype=torch.float16, device="cuda")
    zq.w8a8_gemm_dequant(dev(Xq), dev(s_x), dev(Wq), dev(s_w), G, dev(bias), act,
                         path=zq.PATH_TILED, out=buf[:M * N].view(M, N))
    flat = host(buf)
    assert np.all(flat[M * N:] == 7.0)
    got = flat[:M * N].reshape(M, N)
    assert_y(got, want)
    ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
    off = np.abs(got.astype(np.float64) - want.astype(np.float64)) > ulp
    assert off.mean() <= 1e-3, off.mean()


def test_gemm_no_bias_and_zero_scale_token(zq):
    """A token with scale 0 (all-zero row) gives exactly the bias; without
    bias it gives exactly 0."""
    say("zero-scale token")
    rng = np.random.default_rng(7)
    M, N, K = 40, 64, 64
    Xq = random_int8(rng, (M, K))
    Xq[3] = 0
    Wq = random_int8(rng, (N, K))
    s_x = np.full(M, 0.01, np.float32)
    s_x[3] = 0.0
    s_w = np.full(N // 16, 0.001, np.float32)
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32)
    y = host(zq.w8a8_gemm_dequant(dev(Xq), dev(s_x), dev(Wq), dev(s_w), 16, dev(bias)))
    assert np.array_equal(y[3], bias.astype(np.float16))
    y0 = host(zq.w8a8_gemm_dequant(dev(Xq), dev(s_x), dev(Wq), dev(s_w), 16, None))
    assert not y0[3].any()
    assert_y(y0, ref.epilogue(ref.gemm_i32(Xq, Wq), s_x, s_w, 16, None, 0))


# ---------------------------------------------------------------- prologue

PROLOGUE_CASES = [
    # M, K, pre, x dtype, affine
    (16, 256, ref.PRE_LAYERNORM, np.float32, False),
    (37, 768, ref.PRE_LAYERNORM, np.float16, True),
    (64, 4096, ref.PRE_LAYERNORM, np.float16, False),
    (8, 5120, ref.PRE_LAYERNORM, np.float16, True),
    (5, 8192, ref.PRE_LAYERNORM, np.float32, True),
    (3, 8208, ref.PRE_LAYERNORM, np.float16, True),   # just past the one-wave-per-token limit
    (16, 28672, ref.PRE_GELU, np.float16, False),
    (9, 336, ref.PRE_GELU, np.float32, False),
    (7, 16, ref.PRE_LAYERNORM, np.float16, True),     # smallest K
    (2, 131072, ref.PRE_LAYERNORM, np.float16, False),  # largest K
    # few tokens, long rows: each row spread over ceil(K / 2048) workgroups
    (16, 28672, ref.PRE_GELU, np.float32, False),
    (64, 6160, ref.PRE_GELU, np.float16, False),     # ragged last segment, largest such M
    (65, 4096, ref.PRE_GELU, np.float16, False),     # one more token: one-row-per-wave path
    (3, 4080, ref.PRE_GELU, np.float16, False),      # just below the long-row threshold
    (11, 12304, ref.PRE_LAYERNORM, np.float32, True),
    (1, 131072, ref.PRE_GELU, np.float16, False),
    # fp16 rows of at most 8192 elements and more than 64 tokens (the per-op
    # kernel): each piece count per lane, a last piece holding 2 of 256 chunks,
    # token counts that leave a partial block
    (101, 2048, ref.PRE_LAYERNORM, np.float16, True),   # one wave per token, 4 pieces
    (70, 2064, ref.PRE_LAYERNORM, np.float16, True),    # four waves, 2 pieces, ragged
    (90, 5120, ref.PRE_GELU, np.float16, False),        # 3 pieces
    (67, 6160, ref.PRE_NONE, np.float16, False),        # 4 pieces, ragged
    (130, 8192, ref.PRE_LAYERNORM, np.float16, True),   # 4 whole pieces
    (66, 1040, ref.PRE_NONE, np.float16, False),        # one wave per token, 3 pieces
    (1, 768, ref.PRE_LAYERNORM, np.float16, True),      # one token: three idle waves
    (2, 4080, ref.PRE_NONE, np.float16, False),         # two tokens of four waves each
]


@pytest.mark.parametrize("M,K,pre,dt,affine", PROLOGUE_CASES)
def test_prologue(zq, M, K, pre, dt, affine):
    say("prologue", M, K, pre, dt.__name__, affine)
    rng = np.random.default_rng(M + K + pre)
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(dt)
    g, b = random_affine(rng, K) if affine else (None, None)
    q_ref, s_ref = ref.prologue(X, pre, g, b, 1e-5)
    q, s = zq.ln_quant_per_token(dev(X), pre, None if g is None else dev(g),
                                 None if b is None else dev(b), 1e-5)
    assert_codes(host(q), q_ref)
    assert_scales(host(s), s_ref)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_prologue_gelu_negative_side(zq, dt):
    """Rows whose largest |GeLU| lies on the negative side (around GeLU's
    minimum at x = -0.7518), including rows with no value past the minimum
    and rows with no value before it."""
    say("prologue gelu negative", dt.__name__)
    rng = np.random.default_rng(11)
    M, K = 6, 8192
    X = -3.0 * rng.random((M, K))                      # (-3, 0]
    X[1] = -0.5 * rng.random(K)                        # all in (x0, 0]: R decides
    X[2] = -0.8 - 2.0 * rng.random(K)                  # all below x0: L decides
    X[3, :] = -0.7517915                               # the minimum itself
    X[4] = 0.25 * rng.random(K) - 1.0                  # small positives and negatives
    X[5] = -1e-3 * rng.random(K)                       # tiny values
    X = X.astype(dt)
    q_ref, s_ref = ref.prologue(X, ref.PRE_GELU)
    q, s = zq.ln_quant_per_token(dev(X), ref.PRE_GELU)
    assert_codes(host(q), q_ref)
    assert_scales(host(s), s_ref)


@pytest.mark.parametrize("M,K", [(12, 20000), (1, 4096), (64, 131072)])
def test_prologue_none_long_rows_exact(zq, M, K):
    say("prologue none long", M, K)
    rng = np.random.default_rng(M + K)
    X = (rng.standard_normal((M, K)) * np.exp(2 * rng.standard_normal((M, 1)))).astype(np.float16)
    X[0, :] = 0
    q_ref, s_ref = ref.prologue(X, ref.PRE_NONE)
    q, s = zq.ln_quant_per_token(dev(X), ref.PRE_NONE)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(s), s_ref)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_prologue_none_is_exact(zq, dt):
    """Without a pre-op there is no reduction-order freedom: y = x, the
    absmax is exact and the division is IEEE, so codes and scales are
    identical to the oracle's."""
    say("prologue none", dt.__name__)
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((50, 1040)) * np.exp(2 * rng.standard_normal((50, 1)))).astype(dt)
    X[7] = 0
    q_ref, s_ref = ref.prologue(X, ref.PRE_NONE)
    q, s = zq.ln_quant_per_token(dev(X), zq.PRE_NONE)
    assert_codes(host(q), q_ref, exact=True)
    assert np.array_equal(host(s), s_ref)
    assert host(s)[7] == 0 and not host(q)[7].any()


def test_prologue_golden_halves(zq):
    """Exact half-integer ratios round to even on the GPU too."""
    say("prologue golden halves")
    x = np.zeros((2, 16), np.float32)
    x[0, :8] = [127, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, -127]
    x[1, :6] = [254, 1, 3, -5, -254, 0.9999]
    q, s = zq.ln_quant_per_token(dev(x), zq.PRE_NONE)
    q = host(q)
    assert q[0, :8].tolist() == [127, 0, 2, 2, 0, -2, 126, -127]
    assert q[1, :6].tolist() == [127, 0, 2, -2, -127, 0]
    assert host(s).tolist() == [1.0, 2.0]


# ---------------------------------------------------------------- offline

@pytest.mark.parametrize("N,K,G,dt,smooth", [
    (256, 256, 64, np.float32, False),
    (384, 784, 128, np.float16, False),
    (96, 4096, 1, np.float32, True),
    (64, 160, 64, np.float32, True),
])
def test_weight_quantization_exact(zq, N, K, G, dt, smooth):
    say("wquant", N, K, G, dt.__name__, smooth)
    rng = np.random.default_rng(N + K + G)
    W = (0.02 * rng.standard_normal((N, K)) * np.exp(0.5 * rng.standard_normal((N, 1)))).astype(dt)
    s = np.exp(rng.standard_normal(K)).astype(np.float32) if smooth else None
    Wf = W.astype(np.float32)
    Wsrc = ref.fold_weights(Wf, s) if smooth else Wf
    q_ref, sw_ref = ref.quantize_groups(Wsrc, G)
    q, sw = zq.quantize_weights_grouped(dev(W), G, None if s is None else dev(s))
    assert np.array_equal(host(sw), sw_ref)
    assert_codes(host(q), q_ref, "weight codes", exact=True)


def test_smoothquant_factors(zq):
    say("smoothquant factors")
    rng = np.random.default_rng(21)
    M, K, N = 300, 512, 200
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, rng.choice(K, 5, replace=False)] *= 100
    X = X.astype(np.float16)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    g, b = random_affine(rng, K)
    s_ref = ref.smooth_factors(X, W, 1e-5)
    g_ref, b_ref = ref.fold_ln(g, b, s_ref)
    s, g2, b2 = zq.smoothquant_factors(dev(X), dev(W), 1e-5, dev(g), dev(b))
    s, g2, b2 = host(s), host(g2), host(b2)
    assert_scales(s, s_ref, "smooth")
    # the fold itself is exact given the factor
    assert np.array_equal(g2, (g / s).astype(np.float32))
    assert np.array_equal(b2, (b / s).astype(np.float32))


# ---------------------------------------------------------------- layer

@pytest.mark.parametrize("M", [1, 16, 32, 33, 200])
def test_linear_small(zq, M):
    say("linear", M)
    rng = np.random.default_rng(M)
    K, N, G = 512, 384, 128
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(np.float16)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    g, b = random_affine(rng, K)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    Wq, s_w = ref.quantize_groups(W, G)
    want, _, _ = ref.linear(X, ref.PRE_LAYERNORM, g, b, 1e-5, Wq, s_w, G, bias, ref.ACT_GELU)
    got = host(zq.linear_w8a8(dev(X), dev(Wq), dev(s_w), G, zq.PRE_LAYERNORM, dev(g), dev(b), 1e-5,
                              dev(bias), zq.ACT_GELU))
    assert_y(got, want)


def test_linear_deterministic(zq):
    say("linear determinism")
    rng = np.random.default_rng(5)
    M, K, N, G = 300, 1024, 512, 128
    X = dev(rng.standard_normal((M, K)).astype(np.float16))
    Wq = dev(random_int8(rng, (N, K)))
    s_w = dev(np.full(N // G, 1e-3, np.float32))
    a = host(zq.linear_w8a8(X, Wq, s_w, G))
    b = host(zq.linear_w8a8(X, Wq, s_w, G))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("M,K,pre", [
    (3, 8208, ref.PRE_GELU),      # one segment of 16 elements past the one-wave limit
    (16, 28672, ref.PRE_GELU),    # the decode shape: 14 full segments
    (40, 10000, ref.PRE_NONE),    # ragged last segment, tiled GEMM path
    (5, 131072, ref.PRE_GELU),    # 64 workgroups per row, the largest K
])
def test_linear_long_row_prologue(zq, M, K, pre):
    """Inside zq_linear_w8a8 the codes and scales the prologue leaves in the
    workspace (few tokens with long rows: each row over many workgroups)
    follow the same rules as the standalone prologue's."""
    say("linear prologue", M, K, pre)
    rng = np.random.default_rng(M + K)
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(np.float16)
    N, G = 64, 64
    Wq = random_int8(rng, (N, K))
    s_w = np.full(N // G, 1e-3, np.float32)
    ws = torch.zeros(zq.linear_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    Y = host(zq.linear_w8a8(dev(X), dev(Wq), dev(s_w), G, pre, workspace=ws))
    q_ref, s_ref = ref.prologue(X, pre)
    w = host(ws)
    codes = w[:M * K].view(np.int8).reshape(M, K)
    off = (M * K + 255) // 256 * 256
    scales = w[off:off + 4 * M].view(np.float32)
    assert_codes(codes, q_ref)
    assert_scales(scales, s_ref)
    assert_y(Y, ref.epilogue(ref.gemm_i32(q_ref, Wq), s_ref, s_w, G, None, 0))
