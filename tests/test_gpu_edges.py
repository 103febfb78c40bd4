"""Edge cases of the hot path against the oracle, through the C ABI.

- The int8 GEMM in its int32 test mode, bit-exact, at the layer shapes of the
  workloads (full size; the oracle takes sampled tokens, every output
  column) and at shapes that take each tile configuration, including tile
  counts that are not a multiple of the XCD count, ragged M and N tails and
  a K that ends inside a slab, and where a partly filled last round of
  256 x 256 tiles is split off into a second launch of 128 x 192 tiles (int32
  and the fp16 dequant epilogue).
- LayerNorm of rows whose values are all equal ("探秘Transformer系列之（36）"
  1.2.2: the quantizer follows the LayerNorm; a row of equal values has zero
  variance, so y = beta exactly): codes and scales must equal the oracle's
  exactly, which means scale 0 and codes 0 when beta = 0.
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


def sample_rows(M, rng, edge=64, extra=32):
    """The first and last `edge` tokens (whole first and last row tiles) and
    `extra` tokens drawn at random in between."""
    rows = np.concatenate([np.arange(min(edge, M)), np.arange(max(0, M - edge), M),
                           rng.integers(0, M, extra)])
    return np.unique(rows)


# M, N, K: the workloads' GEMMs (BERT FFN-up and FFN-down, GPT QKV, the outlier
# layer), then ragged shapes: 126 and 731 tiles of 256 x 192 (not multiples of
# 8), a 256 x 256 grid with ragged M and N, and a K ending 16 bytes into a slab.
WORKLOAD_GEMMS = [
    (4096, 3072, 768),
    (4096, 768, 3072),
    (2048, 12288, 4096),
    (4096, 13824, 5120),
    (2304, 2560, 1040),
    (4196, 8180, 512),
    (3000, 5000, 4112),
]


@pytest.mark.parametrize("M,N,K", WORKLOAD_GEMMS)
def test_gemm_int32_workload_shapes(zq, M, N, K):
    say("i32 workload shape", M, N, K)
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    got = host(zq.w8a8_gemm_dequant(dev(Xq), None, dev(Wq), None, 4, out_dtype=torch.int32,
                                    path=zq.PATH_TILED))
    rows = sample_rows(M, rng)
    want = ref.gemm_i32(Xq[rows], Wq)
    bad = np.argwhere(got[rows] != want)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at (row {rows[bad[0][0]]}, col {bad[0][1]})"


# Shapes whose 256 x 256 tiles would leave a last round at most half full, so
# the columns past the last whole round go to a second launch of 128 x 192
# tiles: ragged M, a ragged tail of columns, output rows only 8-byte aligned
# (N % 8 == 4), a K that ends inside a slab, and the weight-group scales and
# bias taken from the middle of their arrays in the second launch.
ROUND_SPLIT = [
    # M, N, K, G
    (1796, 18436, 208, 4),
    (4096, 13312, 1040, 128),
]


@pytest.mark.parametrize("M,N,K,G", ROUND_SPLIT)
def test_gemm_round_split(zq, M, N, K, G):
    say("round split", M, N, K, G)
    rng = np.random.default_rng(M + 5 * N + 11 * K + G)
    Xq = random_int8(rng, (M, K))
    Wq = random_int8(rng, (N, K))
    s_x = (np.exp(rng.standard_normal(M)) * 0.01).astype(np.float32)
    s_w = (np.exp(rng.standard_normal(N // G)) * 2e-4).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    rows = sample_rows(M, rng)
    acc = ref.gemm_i32(Xq[rows], Wq)

    got_i32 = host(zq.w8a8_gemm_dequant(dev(Xq), None, dev(Wq), None, G, out_dtype=torch.int32,
                                        path=zq.PATH_TILED))
    bad = np.argwhere(got_i32[rows] != acc)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at (row {rows[bad[0][0]]}, col {bad[0][1]})"
    del got_i32

    for act in (0, 1):
        want = ref.epilogue(acc, s_x[rows], s_w, G, bias, act)
        guard = 4096
        buf = torch.full((M * N + guard,), 7.0, dtype=torch.float16, device="cuda")
        zq.w8a8_gemm_dequant(dev(Xq), dev(s_x), dev(Wq), dev(s_w), G, dev(bias), act,
                             path=zq.PATH_TILED, out=buf[:M * N].view(M, N))
        flat = host(buf)
        assert np.all(flat[M * N:] == 7.0)
        got = flat[:M * N].reshape(M, N)[rows]
        assert_y(got, want)
        ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
        off = np.abs(got.astype(np.float64) - want.astype(np.float64)) > ulp
        assert off.mean() <= 1e-3, off.mean()


# ---------------------------------------------------------------- constant rows

@pytest.mark.parametrize("dt", [np.float16, np.float32])
@pytest.mark.parametrize("K", [256, 768, 5120, 12304])
@pytest.mark.parametrize("M", [8, 80])
@pytest.mark.parametrize("beta_zero", [True, False])
def test_prologue_constant_rows_layernorm(zq, dt, K, M, beta_zero):
    """Every other token is a row of one repeated value (a different value per
    token, some far from 1 in magnitude); the others are ordinary rows.  With
    M = 8 and K >= 4096 each row is spread over several workgroups, with
    M = 80 one or more waves take a whole row."""
    say("constant rows", dt.__name__, K, M, beta_zero)
    rng = np.random.default_rng(K + M + int(beta_zero))
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(dt)
    const = np.arange(0, M, 2)
    vals = (rng.standard_normal(const.size) * np.exp(3 * rng.standard_normal(const.size)))
    X[const] = vals.astype(dt)[:, None]
    X[const[0]] = dt(0.0)
    g, b = random_affine(rng, K)
    if beta_zero:
        b = np.zeros(K, np.float32)
    q_ref, s_ref = ref.prologue(X, ref.PRE_LAYERNORM, g, b, 1e-5)
    q, s = zq.ln_quant_per_token(dev(X), zq.PRE_LAYERNORM, dev(g), dev(b), 1e-5)
    q, s = host(q), host(s)
    assert_codes(q[const], q_ref[const], "constant-row codes", exact=True)
    assert np.array_equal(s[const], s_ref[const]), (s[const], s_ref[const])
    if beta_zero:
        assert not s[const].any() and not q[const].any()
    other = np.setdiff1d(np.arange(M), const)
    assert_codes(q[other], q_ref[other])
    assert_scales(s[other], s_ref[other])


def test_linear_constant_rows_give_bias(zq):
    """Through the whole layer: a constant token under LayerNorm with beta = 0
    has scale 0 and codes 0, so its output row is exactly fp16(bias)."""
    say("linear constant rows")
    rng = np.random.default_rng(5)
    M, K, N, G = 48, 768, 384, 128
    X = rng.standard_normal((M, K)).astype(np.float16)
    X[[0, 17, 47]] = np.array([[3.25], [-1e-3], [700.0]], dtype=np.float16)
    Wq = random_int8(rng, (N, K))
    s_w = np.full(N // G, 1e-3, np.float32)
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32)
    Y = host(zq.linear_w8a8(dev(X), dev(Wq), dev(s_w), G, zq.PRE_LAYERNORM, None, None, 1e-5,
                            dev(bias)))
    for m in (0, 17, 47):
        assert np.array_equal(Y[m], bias.astype(np.float16)), m


def test_binding_rejects_mismatched_out_and_workspace(zq):
    """out= and workspace= tensors are checked before the call: the C ABI cannot
    see their sizes, so a wrong dtype, shape, device or a short buffer raises
    instead of writing past the end."""
    say("binding out/workspace checks")
    rng = np.random.default_rng(1)
    M, N, K, G = 32, 48, 64, 16
    Xq, Wq = dev(random_int8(rng, (M, K))), dev(random_int8(rng, (N, K)))
    sx = dev(np.full(M, 0.01, np.float32))
    sw = dev(np.full(N // G, 0.01, np.float32))
    with pytest.raises(TypeError):
        zq.w8a8_gemm_dequant(Xq, None, Wq, None, G, out_dtype=torch.int32,
                             out=torch.empty((M, N), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        zq.w8a8_gemm_dequant(Xq, sx, Wq, sw, G,
                             out=torch.empty((M, N - 1), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        zq.w8a8_gemm_dequant(Xq, sx, Wq, sw, G, out=torch.empty((M, N), dtype=torch.float16))
    X = dev(rng.standard_normal((M, K)).astype(np.float16))
    need = zq.linear_workspace_bytes(M, K)
    with pytest.raises(ValueError, match="bytes"):
        zq.linear_w8a8(X, Wq, sw, G, workspace=torch.empty(need - 1, dtype=torch.uint8,
                                                            device="cuda"))
    with pytest.raises(ValueError, match="workspace is on cpu"):
        zq.linear_w8a8(X, Wq, sw, G, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError):
        zq.ln_quant_per_token(X, out=(torch.empty((M, K - 16), dtype=torch.int8, device="cuda"),
                                      torch.empty(M, dtype=torch.float32, device="cuda")))
    # the exact sizes still work
    Y = zq.linear_w8a8(X, Wq, sw, G, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    assert tuple(Y.shape) == (M, N)
