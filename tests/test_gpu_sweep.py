"""A seeded random sweep of the whole layer over its argument space, through
the C ABI, against the oracle.

Each case draws M, K, N, the group size G, the pre-op (none, LayerNorm,
GeLU), the epilogue activation, the input dtype, whether LayerNorm has an
affine and whether there is a bias, and (few tokens) row-major or packed
weights ("探秘Transformer系列之（36）" 1.2.2: per-token activations, group-wise
weights, the INT8 GEMM's INT32 accumulation scaled before the FP16 result).
One call of the layer, then:

- the weight codes and scales the library quantizes equal the oracle's;
- the codes and per-token scales the layer leaves in its workspace follow
  the prologue rules (codes +-1 on at most floor(1e-4 n) near-ties, scales
  within 4 ulps);
- the int32 GEMM on the workspace's own codes is bit-exact;
- Y matches the oracle's layer (max and normwise error bounds), and matches
  the oracle's epilogue applied to the GPU's own codes and scales to 1 fp16
  ulp on all but 1e-3 of the outputs.

The first 24 cases also run the FP8 (E4M3) layer ("探秘Transformer系列之（36）"
ZeroQuant-FP paragraph: FP8 codes with power-of-two scales): weight codes and
scales exact, workspace codes within one code step on near-ties, scales equal
up to 4 ulps, Y within the output tolerance of the oracle's FP8 layer and of
the oracle's product of the GPU's own codes.

The first 20 cases also run the mixed-precision decomposition ("探秘Transformer
系列之（36）" 1.1, LLM.int8(): input channels whose |y| exceeds alpha stay in
fp16, the rest W8A8) on inputs with a seeded set of amplified channels, with
alpha = 6.0 or the nearest listed value that no column maximum sits on: Y
within the output tolerance of the oracle's decomposed layer.

The first 16 cases also run the chained FFN block (the case's K as the model
width, its N rounded up as the hidden width; bit-identical to two layer calls,
and against the oracle's chain) and the unfused order (the ZeroQuant reading
notes' flow before fusion: its codes equal the oracle's quantizer on the GPU's
own fp16 tensor, its int32 accumulators are exact, its output has the fused
epilogue's bits for the same codes, and it matches the oracle's unfused layer).

Every case has at least 10^4 activation codes, and the oracle's integer
products stay under ~1e8 multiply-adds per case, so the sweep runs in
seconds.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

from oracle import ref
from tests._match import assert_codes, assert_fp8_codes, assert_scales, assert_y, say
from zq_workloads import Workload, make_inputs, random_affine

torch = pytest.importorskip("torch")


@dataclasses.dataclass(frozen=True)
class Case:
    seed: int
    M: int
    K: int
    N: int
    G: int
    pre: int
    act: int
    f32: bool
    affine: bool
    bias: bool
    packed: bool

    def __str__(self):
        return (f"s{self.seed}-M{self.M}-K{self.K}-N{self.N}-G{self.G}-pre{self.pre}-act{self.act}"
                f"-{'f32' if self.f32 else 'f16'}{'-aff' if self.affine else ''}"
                f"{'-bias' if self.bias else ''}{'-packed' if self.packed else ''}")


def draw_cases(n: int = 48, seed: int = 20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        few = i % 3 == 0
        M = int(rng.integers(1, 33)) if few else int(rng.integers(33, 700))
        k_lo = -(-10_000 // M // 16)                # at least 10^4 codes
        k_hi = max(k_lo + 1, 768 if few else 320)    # K up to 12272 (few tokens) or 5104
        K = 16 * int(rng.integers(k_lo, k_hi))
        G = int(rng.choice([1, 4, 16, 32, 64, 128]))
        step = int(np.lcm(G, 4))                     # N % G == 0 and N % 4 == 0
        N = step * int(rng.integers(1, max(2, 1024 // step + 1)))
        while M * N * K > 1e8 and N > step:
            N -= step
        cases.append(Case(seed=i, M=M, K=K, N=N, G=G, pre=int(rng.integers(0, 3)),
                          act=int(rng.integers(0, 2)), f32=bool(rng.random() < 0.25),
                          affine=bool(rng.random() < 0.5), bias=bool(rng.random() < 0.6),
                          packed=bool(few and rng.random() < 0.5)))
    return cases


CASES = draw_cases()


@pytest.fixture(scope="module")
def zq():
    import post_w8a8_quantized_amd as m
    assert torch.cuda.is_available(), "a GPU device node exists but torch sees no GPU"
    m.library()
    return m


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_cases_cover_the_argument_space():
    """The drawn cases reach every pre-op, activation, dtype and weight layout,
    both GEMM paths, every group size, and ragged shapes (no GPU needed)."""
    seen = lambda f: {f(c) for c in CASES}
    assert seen(lambda c: c.pre) == {0, 1, 2}
    assert seen(lambda c: c.act) == {0, 1}
    assert seen(lambda c: c.f32) == {False, True}
    assert seen(lambda c: c.packed) == {False, True}
    assert seen(lambda c: c.M <= 32) == {False, True}
    assert seen(lambda c: c.G) == {1, 4, 16, 32, 64, 128}
    assert any(c.M % 128 and c.N % 128 and c.K % 128 for c in CASES)
    assert all(c.M * c.K >= 10_000 for c in CASES)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=str)
def test_layer_sweep(zq, case):
    say("sweep", case)
    c = case
    rng = np.random.default_rng(1000 + c.seed)
    dt = np.float32 if c.f32 else np.float16
    X = (rng.standard_normal((c.M, c.K)) * np.exp(rng.standard_normal((c.M, 1)))).astype(dt)
    W = (0.02 * rng.standard_normal((c.N, c.K)) *
         np.exp(0.5 * rng.standard_normal((c.N, 1)))).astype(np.float32)
    g, b = random_affine(rng, c.K) if c.affine and c.pre == ref.PRE_LAYERNORM else (None, None)
    bias = (0.01 * rng.standard_normal(c.N)).astype(np.float32) if c.bias else None
    eps = 1e-5

    Wq, s_w = ref.quantize_groups(W, c.G)
    Wq_d, sw_d = zq.quantize_weights_grouped(dev(W), c.G)
    assert np.array_equal(host(Wq_d), Wq), "weight codes"
    assert np.array_equal(host(sw_d), s_w), "weight scales"

    ws = torch.zeros(zq.linear_workspace_bytes(c.M, c.K), dtype=torch.uint8, device="cuda")
    if c.packed:
        Y = zq.linear_w8a8_packed(dev(X), zq.pack_weights(Wq_d), sw_d, c.G, c.N, c.pre, dev(g),
                                  dev(b), eps, dev(bias), c.act, workspace=ws)
    else:
        Y = zq.linear_w8a8(dev(X), Wq_d, sw_d, c.G, c.pre, dev(g), dev(b), eps, dev(bias), c.act,
                           workspace=ws)
    Y = host(Y)
    w = host(ws)
    codes = w[:c.M * c.K].view(np.int8).reshape(c.M, c.K)
    off = (c.M * c.K + 255) // 256 * 256
    scales = w[off:off + 4 * c.M].view(np.float32).copy()

    q_ref, sx_ref = ref.prologue(X, c.pre, g, b, eps)
    assert_codes(codes, q_ref)
    assert_scales(scales, sx_ref)

    acc_gpu = host(zq.w8a8_gemm_dequant(dev(codes), None, Wq_d, None, c.G,
                                        out_dtype=torch.int32))
    acc = ref.gemm_i32(codes, Wq)
    bad = np.argwhere(acc_gpu != acc)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at {tuple(bad[0])}"

    assert_y(Y, ref.epilogue(ref.gemm_i32(q_ref, Wq), sx_ref, s_w, c.G, bias, c.act))
    own = ref.epilogue(acc, scales, s_w, c.G, bias, c.act)
    ulp = np.spacing(np.abs(own).astype(np.float16)).astype(np.float64)
    off_ulp = np.abs(Y.astype(np.float64) - own.astype(np.float64)) > ulp
    assert off_ulp.mean() <= 1e-3, f"{off_ulp.sum()} outputs beyond 1 fp16 ulp of the oracle's epilogue"


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES[:24], ids=str)
def test_layer_sweep_fp8(zq, case):
    say("sweep fp8", case)
    c = case
    rng = np.random.default_rng(2000 + c.seed)
    dt = np.float32 if c.f32 else np.float16
    X = (rng.standard_normal((c.M, c.K)) * np.exp(rng.standard_normal((c.M, 1)))).astype(dt)
    W = (0.02 * rng.standard_normal((c.N, c.K)) *
         np.exp(0.5 * rng.standard_normal((c.N, 1)))).astype(np.float32)
    g, b = random_affine(rng, c.K) if c.affine and c.pre == ref.PRE_LAYERNORM else (None, None)
    bias = (0.01 * rng.standard_normal(c.N)).astype(np.float32) if c.bias else None
    eps = 1e-5

    Wq, s_w = ref.quantize_groups_fp8(W, c.G)
    Wq_d, sw_d = zq.quantize_weights_grouped_fp8(dev(W), c.G)
    assert np.array_equal(host(Wq_d), Wq), "FP8 weight codes"
    assert np.array_equal(host(sw_d), s_w), "FP8 weight scales"

    ws = torch.zeros(zq.linear_workspace_bytes(c.M, c.K), dtype=torch.uint8, device="cuda")
    W_arg = zq.pack_weights(Wq_d.view(torch.int8)).view(torch.uint8) if c.packed else Wq_d
    Y = host(zq.linear_w8a8_fp8(dev(X), W_arg, sw_d, c.G, c.pre, dev(g), dev(b), eps, dev(bias),
                                c.act, workspace=ws, N=c.N, packed=c.packed))
    w = host(ws)
    codes = w[:c.M * c.K].reshape(c.M, c.K).copy()
    off = (c.M * c.K + 255) // 256 * 256
    scales = w[off:off + 4 * c.M].view(np.float32).copy()

    q_ref, sx_ref = ref.prologue_fp8(X, c.pre, g, b, eps)
    assert_fp8_codes(codes, q_ref)
    assert_scales(scales, sx_ref)
    assert_y(Y, ref.linear_fp8(X, c.pre, g, b, eps, Wq, s_w, c.G, bias, c.act)[0])
    assert_y(Y, ref.epilogue_f64acc(ref.gemm_fp8(codes, Wq), scales, s_w, c.G, bias, c.act),
             "Y against the oracle's product of the GPU's codes")


DECOMP_ALPHAS = (6.0, 6.5, 5.5, 7.0, 5.0, 7.5)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES[:20], ids=str)
def test_layer_sweep_decomp(zq, case):
    say("sweep decomp", case)
    c = case
    rng = np.random.default_rng(3000 + c.seed)
    frac = min(float(rng.choice([0.002, 0.005, 0.01, 0.02])), 64 / c.K)
    gain = float(rng.choice([8.0, 30.0, 100.0]))
    w = Workload("sweep_decomp", c.M, c.K, c.N, c.G, "f32" if c.f32 else "f16", c.pre, c.act,
                 c.bias, 0.3, 0.02, 0.0, max(frac, 1.0 / c.K), gain, False, seed=3000 + c.seed)
    inp = make_inputs(w)
    # The outlier test |y| > alpha is decided on fp32 y, whose last bits differ
    # between the two sides: take the first alpha (6.0 is LLM.int8()'s) that no
    # column maximum lies within 1e-4 of, so that the set is unambiguous.
    colmax = np.max(np.abs(ref.preop(inp.X, c.pre).astype(np.float64)), axis=0)
    alpha = next(a for a in DECOMP_ALPHAS if not np.any(np.abs(colmax - a) <= 1e-4 * a))
    Wq_r, s_w_r = ref.quantize_groups(inp.W, c.G)
    want, _, _, cols = ref.linear_decomp(inp.X, c.pre, None, None, 1e-5, alpha, Wq_r,
                                         s_w_r, c.G, inp.W, inp.bias, c.act)
    assert cols.size > 0
    Wd = dev(inp.W)
    Wq, s_w = zq.quantize_weights_grouped(Wd, c.G)
    got = zq.linear_w8a8_decomp(dev(inp.X), Wq, s_w, c.G, zq.pack_outlier_weights(Wd),
                                alpha, c.pre, bias=dev(inp.bias), act=c.act)
    assert_y(host(got), want)


def r256(v):
    return (v + 255) // 256 * 256


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES[:16], ids=str)
def test_ffn_sweep(zq, case):
    say("sweep ffn", case)
    c = case
    rng = np.random.default_rng(4000 + c.seed)
    K = c.K
    F = -(-c.N // int(np.lcm(c.G, 16))) * int(np.lcm(c.G, 16))   # F % G1 == 0, F % 16 == 0
    while c.M * F * K > 5e7 and K > 16:
        K = max(16, K // 2 // 16 * 16)
    G1, G2 = c.G, 16
    dt = np.float32 if c.f32 else np.float16
    X = (rng.standard_normal((c.M, K)) * np.exp(rng.standard_normal((c.M, 1)))).astype(dt)
    g, b = random_affine(rng, K)
    W1 = (0.02 * rng.standard_normal((F, K))).astype(np.float32)
    W2 = (0.02 * rng.standard_normal((K, F))).astype(np.float32)
    b1 = (0.01 * rng.standard_normal(F)).astype(np.float32)
    b2 = (0.01 * rng.standard_normal(K)).astype(np.float32)
    W1q, s1 = zq.quantize_weights_grouped(dev(W1), G1)
    W2q, s2 = zq.quantize_weights_grouped(dev(W2), G2)
    Xd, gd, bd, b1d, b2d = dev(X), dev(g), dev(b), dev(b1), dev(b2)
    ws = torch.zeros(zq.ffn_workspace_bytes(c.M, K, F), dtype=torch.uint8, device="cuda")
    Y = host(zq.ffn_w8a8(Xd, W1q, s1, G1, W2q, s2, G2, gd, bd, 1e-5, b1d, b2d, workspace=ws))
    H2 = zq.linear_w8a8(Xd, W1q, s1, G1, zq.PRE_LAYERNORM, gd, bd, 1e-5, b1d, zq.ACT_GELU)
    Y2 = host(zq.linear_w8a8(H2, W2q, s2, G2, zq.PRE_NONE, None, None, 1e-5, b2d, zq.ACT_NONE))
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16)), "chain != two layer calls"
    W1q_h, s1_h, W2q_h, s2_h = host(W1q), host(s1), host(W2q), host(s2)
    H_ref = ref.linear(X, ref.PRE_LAYERNORM, g, b, 1e-5, W1q_h, s1_h, G1, b1, ref.ACT_GELU)[0]
    Y_ref = ref.linear(H_ref, ref.PRE_NONE, None, None, 1e-5, W2q_h, s2_h, G2, b2,
                       ref.ACT_NONE)[0]
    assert_y(Y, Y_ref)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES[:16], ids=str)
def test_unfused_sweep(zq, case):
    say("sweep unfused", case)
    c = case
    rng = np.random.default_rng(5000 + c.seed)
    dt = np.float32 if c.f32 else np.float16
    X = (rng.standard_normal((c.M, c.K)) * np.exp(rng.standard_normal((c.M, 1)))).astype(dt)
    g, b = random_affine(rng, c.K) if c.affine and c.pre == ref.PRE_LAYERNORM else (None, None)
    W = (0.02 * rng.standard_normal((c.N, c.K))).astype(np.float32)
    bias = (0.01 * rng.standard_normal(c.N)).astype(np.float32) if c.bias else None
    Wq, s_w = ref.quantize_groups(W, c.G)
    M, N, K = c.M, c.N, c.K
    ws = torch.zeros(zq.linear_unfused_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    Y = host(zq.linear_w8a8_unfused(dev(X), dev(Wq), dev(s_w), c.G, c.pre, dev(g), dev(b), 1e-5,
                                    dev(bias), c.act, workspace=ws))
    w = host(ws)
    o = 0
    y16 = w[o:o + 2 * M * K].view(np.float16).reshape(M, K)
    o += r256(2 * M * K)
    q = w[o:o + M * K].view(np.int8).reshape(M, K)
    o += r256(M * K)
    sx = w[o:o + 4 * M].view(np.float32).copy()
    o += r256(4 * M)
    acc = w[o:o + 4 * M * N].view(np.int32).reshape(M, N)
    q_own, s_own = ref.quantize_rows(y16.astype(np.float32))
    assert_codes(q, q_own, exact=True)
    assert np.array_equal(sx, s_own)
    assert np.array_equal(acc, ref.gemm_i32(q, Wq))
    Yf = host(zq.w8a8_gemm_dequant(dev(q), dev(sx), dev(Wq), dev(s_w), c.G, dev(bias), c.act))
    assert np.array_equal(Y.view(np.uint16), Yf.view(np.uint16)), "unfused != fused epilogue"
    q_ref, s_ref = ref.unfused_prologue(X, c.pre, g, b, 1e-5)
    assert_y(Y, ref.epilogue(ref.gemm_i32(q_ref, Wq), s_ref, s_w, c.G, bias, c.act))
