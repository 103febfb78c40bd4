"""Pins of the CPU oracle against what the pages and mathematics fix.

Each `pin_*` function raises AssertionError when the oracle disagrees with a
hand-worked example (tests/golden), a closed form, an invariant, a library
routine that the case reduces to, or brute force.  The tests below run every
pin against the oracle; test_oracle_mutants.py runs them against copies of
the oracle with planted mistakes and checks that each mistake is caught.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

from oracle import brute, ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _golden_kv(name):
    out = {}
    for line in _golden_lines(name):
        k, v = line.split(":", 1)
        out[k.strip()] = [float(t) for t in v.split()]
    return out


# --------------------------------------------------------------------------
# Hand-worked examples (tests/golden, each file cites its passage)
# --------------------------------------------------------------------------

def pin_golden_absmax():
    for line in _golden_lines("absmax_quantize.txt"):
        xs, s, qs = (p.strip() for p in line.split("|"))
        x = np.array([[float(t) for t in xs.split()]], dtype=np.float32)
        q, sc = ref.quantize_rows(x)
        assert sc[0] == np.float32(float(s)), (line, sc)
        assert q[0].tolist() == [int(t) for t in qs.split()], (line, q)


def pin_golden_layernorm():
    for line in _golden_lines("layernorm_quantize.txt"):
        xs, qs = (p.strip() for p in line.split("|"))
        x = np.array([[float(t) for t in xs.split()]], dtype=np.float32)
        q, _ = ref.prologue(x, ref.PRE_LAYERNORM, eps=0.0)
        assert q[0].tolist() == [int(t) for t in qs.split()], (line, q)


def pin_golden_gelu():
    for line in _golden_lines("gelu_values.txt"):
        xs, ys = (p.strip() for p in line.split("|"))
        y = ref.preop(np.array([[float(xs)]], dtype=np.float32), ref.PRE_GELU)[0, 0]
        assert abs(float(y) - float(ys)) <= 1e-7 * max(1.0, abs(float(ys))), (line, y)


def pin_golden_fp16():
    for line in _golden_lines("fp16_rounding.txt"):
        vs, hs = (p.strip() for p in line.split("|"))
        got = int(ref.f64_to_f16_bits([float(vs)])[0])
        assert got == int(hs, 16), (line, hex(got))


def pin_golden_linear_integer():
    g = _golden_kv("linear_integer.txt")
    X = np.array([g["x"]], dtype=np.float32)
    W = np.array([g["w0"], g["w1"]], dtype=np.float32)
    bias = np.array(g["bias"], dtype=np.float32)
    Wq, s_w = ref.quantize_groups(W, 2)
    assert s_w.tolist() == [1.0]
    assert np.array_equal(Wq, W.astype(np.int8))
    Y, Xq, s_x = ref.linear(X, ref.PRE_NONE, None, None, 1e-5, Wq, s_w, 2, bias, ref.ACT_NONE)
    assert s_x.tolist() == [1.0]
    assert ref.gemm_i32(Xq, Wq)[0].tolist() == [int(v) for v in g["acc"]]
    assert Y.astype(np.float64)[0].tolist() == g["y"], Y


def pin_golden_smooth():
    g = _golden_kv("smooth_factors.txt")
    X = np.array([g["x0"], g["x1"]], dtype=np.float32)
    W = np.array([g["w0"]], dtype=np.float32)
    s = ref.smooth_factors(X, W, eps=0.0)
    np.testing.assert_allclose(s, g["s"], rtol=2e-7)


# --------------------------------------------------------------------------
# Format facts, brute force and library routines
# --------------------------------------------------------------------------

def pin_fp16_matches_numpy():
    """One RNE rounding binary64 -> binary16, against numpy's own conversion,
    on random values across the range and on exact midpoints."""
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000),
        # exact midpoints between consecutive fp16 values (ties)
        (np.arange(-2000, 2000, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** -10,
        (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** 5,
    ])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    got = ref.f64_to_f16_bits(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(v[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def pin_f16_decode_all_codes():
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    want = h.view(np.float16).astype(np.float32)
    got = ref.f16_bits_to_f32(h)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(want[~np.isnan(want)]))


def _brute_case(seed, M, K, N, G, pre, act, x_dtype, affine, with_bias):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(x_dtype)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    gamma = beta = None
    if affine:
        gamma = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
        beta = (0.1 * rng.standard_normal(K)).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32) if with_bias else None
    return X, W, gamma, beta, bias


BRUTE_CASES = [
    # seed, M, K, N, G, pre, act, x dtype, affine LN, bias
    (0, 3, 16, 4, 2, ref.PRE_LAYERNORM, ref.ACT_NONE, np.float32, False, True),
    (1, 4, 32, 6, 3, ref.PRE_LAYERNORM, ref.ACT_GELU, np.float16, True, True),
    (2, 2, 48, 4, 4, ref.PRE_GELU, ref.ACT_NONE, np.float16, False, False),
    (3, 5, 16, 8, 1, ref.PRE_NONE, ref.ACT_GELU, np.float32, False, True),
    (4, 1, 64, 2, 2, ref.PRE_LAYERNORM, ref.ACT_NONE, np.float16, True, False),
]


def pin_brute_force():
    """The C oracle and the pure-Python brute force agree bit for bit on
    codes, scales and accumulators, and on the fp16 output."""
    for seed, M, K, N, G, pre, act, dt, affine, with_bias in BRUTE_CASES:
        X, W, gamma, beta, bias = _brute_case(seed, M, K, N, G, pre, act, dt, affine, with_bias)
        bq, bs, bwq, bsw, bacc, bY = brute.linear(X, pre, gamma, beta, 1e-5, W, G, bias, act)
        Wq, s_w = ref.quantize_groups(W, G)
        Xq, s_x = ref.prologue(X, pre, gamma, beta, 1e-5)
        acc = ref.gemm_i32(Xq, Wq)
        Y = ref.epilogue(acc, s_x, s_w, G, bias, act)
        assert np.array_equal(Xq, bq) and np.array_equal(s_x, bs), seed
        assert np.array_equal(Wq, bwq) and np.array_equal(s_w, bsw), seed
        assert np.array_equal(acc.astype(np.int64), bacc), seed
        assert np.array_equal(Y.view(np.uint16), bY.view(np.uint16)), seed


def pin_layernorm_matches_torch():
    """LayerNorm reduces to torch.nn.functional.layer_norm evaluated in fp64."""
    import torch
    rng = np.random.default_rng(5)
    for K, affine in [(256, False), (768, True), (1000, True)]:
        X = (rng.standard_normal((8, K)) * np.exp(rng.standard_normal((8, 1)))).astype(np.float32)
        g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32) if affine else None
        b = (0.1 * rng.standard_normal(K)).astype(np.float32) if affine else None
        want = torch.nn.functional.layer_norm(
            torch.from_numpy(X.astype(np.float64)), (K,),
            None if g is None else torch.from_numpy(g.astype(np.float64)),
            None if b is None else torch.from_numpy(b.astype(np.float64)), eps=1e-5).numpy()
        got = ref.preop(X, ref.PRE_LAYERNORM, g, b, 1e-5).astype(np.float64)
        ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - want) <= ulp), np.max(np.abs(got - want) / ulp)


def pin_gelu_matches_torch():
    """GeLU reduces to torch.nn.functional.gelu(approximate='none') in fp64."""
    import torch
    rng = np.random.default_rng(6)
    X = (3.0 * rng.standard_normal((4, 512))).astype(np.float32)
    want = torch.nn.functional.gelu(torch.from_numpy(X.astype(np.float64)), approximate="none").numpy()
    got = ref.preop(X, ref.PRE_GELU).astype(np.float64)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp + 1e-30)


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------

def pin_rounding_error_bound():
    """|y - s q| <= s/2 up to the fp32 rounding of y/s, and no clipping:
    absmax scaling covers the range, so each nonzero row has a code of +-127."""
    rng = np.random.default_rng(7)
    Y = (rng.standard_normal((64, 300)) * np.exp(2 * rng.standard_normal((64, 1)))).astype(np.float32)
    q, s = ref.quantize_rows(Y)
    err = np.abs(Y.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -17))
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    a = np.max(np.abs(Y), axis=1)
    assert np.array_equal(s, (a / np.float32(127)).astype(np.float32))


def pin_power_of_two_scaling():
    """Scaling a token by 2^k scales s by 2^k and leaves codes unchanged;
    LayerNorm with eps = 0 removes the factor exactly."""
    rng = np.random.default_rng(8)
    Y = rng.standard_normal((16, 96)).astype(np.float32)
    q1, s1 = ref.quantize_rows(Y)
    q2, s2 = ref.quantize_rows(Y * np.float32(2.0 ** 7))
    assert np.array_equal(q1, q2) and np.array_equal(s2, s1 * np.float32(2.0 ** 7))
    l1, _ = ref.prologue(Y, ref.PRE_LAYERNORM, eps=0.0)
    l2, _ = ref.prologue(Y * np.float32(2.0 ** -5), ref.PRE_LAYERNORM, eps=0.0)
    assert np.array_equal(l1, l2)


def _numpy_absmax(v: np.ndarray, axis):
    a = np.max(np.abs(v), axis=axis, keepdims=True)
    s = (a / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.clip(np.rint(v / s), -127, 127), 0).astype(np.int8)
    return q, s


def pin_group_special_cases():
    """G = N is per-tensor quantization; G = 1 is per-row (vector-wise)
    quantization; an intermediate G takes each block of G output rows."""
    rng = np.random.default_rng(9)
    W = (0.02 * rng.standard_normal((12, 40)) * np.exp(rng.standard_normal((12, 1)))).astype(np.float32)
    q, s = ref.quantize_groups(W, 12)
    qt, st = _numpy_absmax(W, None)
    assert np.array_equal(q, qt) and s[0] == st.ravel()[0]
    q, s = ref.quantize_groups(W, 1)
    qr, sr = _numpy_absmax(W, 1)
    assert np.array_equal(q, qr) and np.array_equal(s, sr.ravel())
    q, s = ref.quantize_groups(W, 4)
    for g in range(3):
        qg, sg = _numpy_absmax(W[4 * g:4 * g + 4], None)
        assert np.array_equal(q[4 * g:4 * g + 4], qg) and s[g] == sg.ravel()[0]


def pin_gemm_exact():
    """The int GEMM equals numpy's int64 matmul (non-square, so a transposed
    operand shows), and overflow past int32 is reported."""
    rng = np.random.default_rng(10)
    Xq = rng.integers(-127, 128, (9, 200)).astype(np.int8)
    Wq = rng.integers(-127, 128, (13, 200)).astype(np.int8)
    acc = ref.gemm_i32(Xq, Wq)
    assert np.array_equal(acc.astype(np.int64), Xq.astype(np.int64) @ Wq.astype(np.int64).T)
    big = np.full((1, 140000), 127, dtype=np.int8)
    try:
        ref.gemm_i32(big, big)
    except ref.OracleError:
        pass
    else:
        raise AssertionError("int32 overflow not reported")


def pin_epilogue_outer_product():
    """v = s_x[m] s_w[n // G] acc + b equals the fake-quant form
    sum_k (s_x q)(s_w w) + b, and Y is v rounded once to fp16."""
    rng = np.random.default_rng(11)
    M, N, K, G = 6, 512, 64, 128
    Xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s_x = np.exp(rng.standard_normal(M)).astype(np.float32) * np.float32(0.01)
    s_w = np.exp(rng.standard_normal(N // G)).astype(np.float32) * np.float32(1e-3)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    acc = ref.gemm_i32(Xq, Wq)
    for act in (ref.ACT_NONE, ref.ACT_GELU):
        Y, Y64 = ref.epilogue(acc, s_x, s_w, G, bias, act, return_f64=True)
        fq = (s_x[:, None].astype(np.float64) * Xq) @ (np.repeat(s_w, G)[:, None].astype(np.float64) * Wq).T
        v = fq + bias.astype(np.float64)
        if act == ref.ACT_GELU:
            v = 0.5 * v * (1.0 + np.vectorize(math.erf)(v / math.sqrt(2.0)))
        np.testing.assert_allclose(Y64, v, rtol=1e-12, atol=1e-15)
        assert np.array_equal(Y.view(np.uint16), Y64.astype(np.float16).view(np.uint16))


def pin_zero_token():
    """An all-zero token (pre-op NONE) gets scale 0, codes 0 and output = bias."""
    X = np.zeros((2, 32), dtype=np.float32)
    X[1, 3] = 1.0
    Xq, s_x = ref.prologue(X, ref.PRE_NONE)
    assert s_x[0] == 0 and not Xq[0].any() and s_x[1] > 0
    Wq = np.ones((2, 32), dtype=np.int8)
    bias = np.array([0.25, -0.5], dtype=np.float32)
    Y = ref.epilogue(ref.gemm_i32(Xq, Wq), s_x, np.array([1.0], np.float32), 2, bias)
    assert Y[0].astype(np.float32).tolist() == [0.25, -0.5]


def pin_smoothquant_identity():
    """(X diag(s)^-1)(diag(s) W) = X W to 1e-5 relative (max norm) with the
    factors rounded to fp32; after the fold each channel's activation and
    weight maxima are both sqrt(a_j w_j); LN with gamma/s, beta/s is LN / s."""
    rng = np.random.default_rng(12)
    M, K, N = 64, 128, 96
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, [5, 77]] *= np.float32(100.0)
    X = X.astype(np.float16)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    s = ref.smooth_factors(X, W)
    Xt = ref.preop(X, ref.PRE_LAYERNORM)
    Xh = (Xt / s).astype(np.float32)
    Wh = ref.fold_weights(W, s)
    Y0 = Xt.astype(np.float64) @ W.astype(np.float64).T
    Y1 = Xh.astype(np.float64) @ Wh.astype(np.float64).T
    assert np.max(np.abs(Y1 - Y0)) <= 1e-5 * np.max(np.abs(Y0))
    a = np.max(np.abs(Xt), axis=0).astype(np.float64)
    w = np.max(np.abs(W), axis=0).astype(np.float64)
    target = np.sqrt(a * w)
    np.testing.assert_allclose(np.max(np.abs(Xh), axis=0), target, rtol=1e-6)
    np.testing.assert_allclose(np.max(np.abs(Wh), axis=0), target, rtol=1e-6)
    gamma = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(K)).astype(np.float32)
    g2, b2 = ref.fold_ln(gamma, beta, s)
    lhs = ref.preop(X, ref.PRE_LAYERNORM, g2, b2).astype(np.float64)
    rhs = ref.preop(X, ref.PRE_LAYERNORM, gamma, beta).astype(np.float64) / s
    assert np.max(np.abs(lhs - rhs)) <= 1e-6 * np.max(np.abs(rhs))


def pin_round_to_f16_against_numpy():
    """fp32 -> binary16 (nearest even) -> fp32 against numpy's own conversion,
    over normal, subnormal, overflowing and exactly-halfway values."""
    rng = np.random.default_rng(21)
    y = (rng.standard_normal(20000) * np.exp(3 * rng.standard_normal(20000))).astype(np.float32)
    ties = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -24 * 1.5, 2.0 ** -24 * 0.5,
                     65504.0 + 16.0, 65504.0 + 15.99, -(1 + 2.0 ** -11), 6.1e-5], dtype=np.float32)
    y = np.concatenate([y, ties])
    with np.errstate(over="ignore"):
        want = y.astype(np.float16).astype(np.float32)
    assert np.array_equal(ref.round_to_f16(y), want)


def pin_unfused_prologue_reduces_to_fused():
    """Without an op on fp16 input, the FP16 round trip changes nothing: the
    unfused quantizer equals the fused one exactly."""
    rng = np.random.default_rng(22)
    X = (rng.standard_normal((9, 200)) * np.exp(rng.standard_normal((9, 1)))).astype(np.float16)
    qa, sa = ref.unfused_prologue(X, ref.PRE_NONE)
    qb, sb = ref.prologue(X, ref.PRE_NONE)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


def pin_unfused_prologue_brute_force():
    """LN and GeLU, rounded to FP16 between the op and the quantizer, against
    the pure-Python brute force with numpy's float16 rounding in between."""
    rng = np.random.default_rng(23)
    X = (rng.standard_normal((5, 48)) * 3).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(48)).astype(np.float32)
    b = (0.1 * rng.standard_normal(48)).astype(np.float32)
    for pre, gg, bb in ((ref.PRE_LAYERNORM, g, b), (ref.PRE_GELU, None, None)):
        q, s = ref.unfused_prologue(X, pre, gg, bb)
        for m in range(X.shape[0]):
            y = brute.preop_row(X[m], pre, gg, bb)
            y16 = [float(np.float32(v).astype(np.float16)) for v in y]
            qb, sb = brute.quantize_vec(y16)
            assert list(q[m]) == qb and float(s[m]) == sb


def _golden_e4m3():
    dec, enc = [], []
    for line in open(os.path.join(GOLDEN, "e4m3_values.txt"), encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b = (t.strip() for t in line.split("|"))
        if a.startswith("="):
            enc.append((float(a[1:]), int(b, 16)))
        else:
            dec.append((int(a, 16), float(b)))
    return dec, enc


def pin_e4m3_golden():
    """E4M3 codes <-> values from the format definition, incl. ties to even."""
    dec, enc = _golden_e4m3()
    for c, v in dec:
        got = ref.e4m3_to_f64([c])[0]
        assert (np.isnan(v) and np.isnan(got)) or (got == v and np.signbit(got) == np.signbit(v)), c
    for v, c in enc:
        assert ref.f64_to_e4m3([v])[0] == c, v


def pin_e4m3_against_torch():
    """All 256 codes decoded, and fp32 values (random, ties, subnormals, up to 448)
    encoded, against torch's own float8_e4m3fn conversion."""
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ref.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    rng = np.random.default_rng(31)
    v = (rng.standard_normal(5000) * np.exp(2 * rng.standard_normal(5000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    mids = ((want[:126] + want[1:127]) / 2).astype(np.float32)   # exact midpoints
    v = np.concatenate([v, mids, -mids]).astype(np.float32)
    tw = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref.f64_to_e4m3(v.astype(np.float64)), tw)


def pin_pow2_scale_properties():
    """s = 2^e is a power of two, a <= 448 s, and s / 2 would clip (a > 224 s)."""
    rng = np.random.default_rng(32)
    for a in np.concatenate([np.exp(rng.uniform(-30, 30, 500)), [448.0, 448.00003, 1.0, 224.0]]):
        a = float(np.float32(a))
        s = ref.pow2_scale(a)
        m, e = math.frexp(s)
        assert m == 0.5, (a, s)
        assert a <= 448.0 * s and a > 224.0 * s, (a, s)
    assert ref.pow2_scale(0.0) == 0.0


def pin_fp8_quantizer_brute_force():
    """Each code is the nearest E4M3 value to y / s (ties to even), found by
    searching all finite codes; the absmax element lands in (224, 448]."""
    rng = np.random.default_rng(33)
    Y = (rng.standard_normal((4, 64)) * np.exp(rng.standard_normal((4, 1)) * 3)).astype(np.float32)
    Y[3] = 0
    q, s = ref.quantize_rows_fp8(Y)
    vals = ref.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    fin = [c for c in range(256) if not np.isnan(vals[c])]
    for m in range(4):
        if s[m] == 0:
            assert np.all(q[m] == 0)
            continue
        for k in range(64):
            t = float(Y[m, k]) / float(s[m])
            best = min(fin, key=lambda c: (abs(vals[c] - t), (c & 1), c >= 128))
            assert abs(vals[q[m, k]] - t) == abs(vals[best] - t), (m, k)
            if abs(vals[q[m, k]] - t) == abs(vals[best] - t) and vals[q[m, k]] != vals[best]:
                assert q[m, k] & 1 == 0          # a tie goes to the even code
        assert 224.0 < np.max(np.abs(vals[q[m]])) <= 448.0


def pin_fp8_gemm_exact_sums():
    """fp64 accumulation of E4M3 products against exact rational sums."""
    from fractions import Fraction
    rng = np.random.default_rng(34)
    Xq = rng.integers(0, 256, (3, 40)).astype(np.uint8)
    Wq = rng.integers(0, 256, (5, 40)).astype(np.uint8)
    Xq[(Xq & 0x7F) == 0x7F] = 0
    Wq[(Wq & 0x7F) == 0x7F] = 0
    acc = ref.gemm_fp8(Xq, Wq)
    vals = ref.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    for m in range(3):
        for n in range(5):
            exact = sum(Fraction(vals[a]) * Fraction(vals[b]) for a, b in zip(Xq[m], Wq[n]))
            assert acc[m, n] == float(exact)


def pin_fp8_epilogue_reduces_to_int_epilogue():
    """On integer-valued accumulators the fp64-accumulator epilogue equals the
    int32 one exactly."""
    rng = np.random.default_rng(35)
    acc = rng.integers(-100000, 100000, (7, 32)).astype(np.int32)
    s_x = (np.exp(rng.standard_normal(7)) * 0.01).astype(np.float32)
    s_w = (np.exp(rng.standard_normal(4)) * 1e-3).astype(np.float32)
    b = (0.1 * rng.standard_normal(32)).astype(np.float32)
    for act in (ref.ACT_NONE, ref.ACT_GELU):
        a = ref.epilogue(acc, s_x, s_w, 8, b, act)
        c = ref.epilogue_f64acc(acc.astype(np.float64), s_x, s_w, 8, b, act)
        assert np.array_equal(a.view(np.uint16), c.view(np.uint16))


# --------------------------------------------------------------------------
# LLM.int8() mixed-precision decomposition ("探秘Transformer系列之（36）" 1.1)
# --------------------------------------------------------------------------

def _decomp_case(seed, M, K, N, n_out, scale=40.0, x_dtype=np.float32):
    """Tokens N(0,1) with n_out fixed columns scaled up (the outlier pattern
    the page describes: a few systematic feature dimensions)."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    cols = np.sort(rng.choice(K, n_out, replace=False))
    X[:, cols] *= scale
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    return X.astype(x_dtype), W, bias, cols


def pin_decomp_no_outliers_is_fused_layer():
    """With alpha above every |y| the set O is empty and the decomposed layer
    is the fused W8A8 layer, bit for bit."""
    for seed, pre, act, G in ((40, ref.PRE_LAYERNORM, ref.ACT_NONE, 1),
                              (41, ref.PRE_GELU, ref.ACT_GELU, 4),
                              (42, ref.PRE_NONE, ref.ACT_NONE, 2)):
        X, W, bias, _ = _decomp_case(seed, 6, 64, 8, 2)
        Wq, s_w = ref.quantize_groups(W, G)
        Yd, q, s, cols = ref.linear_decomp(X, pre, None, None, 1e-5, 1e30, Wq, s_w, G, W, bias, act)
        Yf, qf, sf = ref.linear(X, pre, None, None, 1e-5, Wq, s_w, G, bias, act)
        assert cols.size == 0
        assert np.array_equal(q, qf) and np.array_equal(s, sf)
        assert np.array_equal(Yd.view(np.uint16), Yf.view(np.uint16))


def pin_decomp_all_outliers_is_fp16_matmul():
    """With alpha below 0 every column is in O: no INT8 part is left (codes and
    scales 0) and the result is the FP16 matmul fp16(y) fp16(W)^T + b, here
    evaluated with numpy's fp16 casts and a float64 matmul."""
    from scipy.special import erf
    X, W, bias, _ = _decomp_case(43, 5, 96, 12, 3)
    for act in (ref.ACT_NONE, ref.ACT_GELU):
        Wq, s_w = ref.quantize_groups(W, 3)
        (Yd, Y64), q, s, cols = ref.linear_decomp(X, ref.PRE_LAYERNORM, None, None, 1e-5, -1.0, Wq,
                                                  s_w, 3, W, bias, act, return_f64=True)
        assert np.array_equal(cols, np.arange(96))
        assert not q.any() and not s.any()
        y = ref.preop(X, ref.PRE_LAYERNORM).astype(np.float16).astype(np.float64)
        w = W.astype(np.float16).astype(np.float64)
        want = y @ w.T + bias.astype(np.float64)
        mag = np.abs(y) @ np.abs(w).T + np.abs(bias)
        if act == ref.ACT_GELU:
            want = 0.5 * want * (1.0 + erf(want / np.sqrt(2.0)))
        assert np.all(np.abs(Y64 - want) <= 1e-12 * mag)


def pin_decomp_outlier_set():
    """O is exactly the planted columns; the test is on magnitude and strict:
    a column whose largest |y| is exactly alpha stays out, the next float
    above alpha (or a negative value below -alpha) is in."""
    rng = np.random.default_rng(44)
    Y = rng.uniform(-5.9, 5.9, (9, 40)).astype(np.float32)
    Y[3, 7] = 6.5
    Y[0, 11] = -6.5
    Y[8, 20] = np.float32(6.0)
    Y[5, 21] = np.nextafter(np.float32(6.0), np.float32(np.inf))
    Y[2, 33] = -np.nextafter(np.float32(6.0), np.float32(np.inf))
    assert np.array_equal(ref.outlier_columns(Y, 6.0), [7, 11, 21, 33])
    assert ref.outlier_columns(Y, 1e9).size == 0
    assert np.array_equal(ref.outlier_columns(Y, -1.0), np.arange(40))


def pin_decomp_quantizer_skips_outlier_columns():
    """Quantizing outside O equals quantizing the row with the O columns set
    to 0 (the absmax and every other code are unchanged by a zero), and the
    codes in O are 0.  The outlier carries the row's absmax here, so counting
    it would change the scale."""
    X, _, _, cols = _decomp_case(45, 7, 80, 4, 3)
    Y = ref.preop(X, ref.PRE_LAYERNORM)
    q, s = ref.quantize_rows_excluding(Y, cols)
    Z = Y.copy()
    Z[:, cols] = 0.0
    qz, sz = ref.quantize_rows(Z)
    assert np.array_equal(q, qz) and np.array_equal(s, sz)
    assert not q[:, cols].any()
    _, s_all = ref.quantize_rows(Y)
    assert np.all(s < s_all)


def pin_decomp_error_bound():
    """Against the unquantized layer in fp64: each INT8 operand is within half
    a step of its value ("Integer Quantization: Deep Dive", 量化误差), each
    FP16 operand within half an fp16 ulp, so
      |Y - Y_float| <= sum_{j not in O} (s_x/2 |w| + |y| s_w/2 + s_x s_w/4)
                       + sum_{j in O} (|y - y16| |w16| + |y| |w - w16|)
    before the output rounding (act = none, compared in fp64)."""
    X, W, bias, planted = _decomp_case(46, 8, 128, 16, 4)
    G = 4
    Wq, s_w = ref.quantize_groups(W, G)
    (Yd, Y64), q, s_x, cols = ref.linear_decomp(X, ref.PRE_LAYERNORM, None, None, 1e-5, 6.0, Wq,
                                                s_w, G, W, bias, ref.ACT_NONE, return_f64=True)
    assert np.array_equal(cols, planted)
    y = ref.preop(X, ref.PRE_LAYERNORM).astype(np.float64)
    w = W.astype(np.float64)
    want = y @ w.T + bias
    inl = np.setdiff1d(np.arange(128), cols)
    sw_n = np.repeat(s_w.astype(np.float64), G)
    sx = s_x.astype(np.float64)[:, None]
    b_int = (sx / 2) * np.abs(w[:, inl]).sum(1)[None, :] + np.abs(y[:, inl]).sum(1)[:, None] * sw_n / 2 \
        + inl.size * sx * sw_n / 4
    y16 = y[:, cols].astype(np.float16).astype(np.float64)
    w16 = w[:, cols].astype(np.float16).astype(np.float64)
    b_out = np.abs(y[:, cols] - y16) @ np.abs(w16).T + np.abs(y[:, cols]) @ np.abs(w[:, cols] - w16).T
    err = np.abs(Y64 - want)
    assert np.all(err <= (b_int + b_out) * (1 + 1e-6) + 1e-12)
    # the outlier columns carry most of the output here: dropping them breaks the bound
    assert np.max(np.abs(y[:, cols] @ w[:, cols].T)) > 10 * np.max(b_int + b_out)


def pin_decomp_brute_force():
    """The C oracle and the pure-Python brute force agree on the outlier set,
    codes and scales exactly and on the fp16 output bit for bit."""
    # (LayerNorm bounds every |y| by sqrt(K - 1), so its case needs K > 37 and
    # a column that dominates the row's variance.)
    for seed, M, K, N, G, pre, act, n_out, sc, dt in (
            (47, 4, 64, 6, 2, ref.PRE_LAYERNORM, ref.ACT_NONE, 1, 40.0, np.float32),
            (48, 3, 32, 4, 1, ref.PRE_GELU, ref.ACT_GELU, 3, 8.0, np.float16),
            (49, 5, 16, 8, 4, ref.PRE_NONE, ref.ACT_NONE, 1, 8.0, np.float32)):
        X, W, bias, _ = _decomp_case(seed, M, K, N, n_out, scale=sc, x_dtype=dt)
        Wq, s_w = ref.quantize_groups(W, G)
        Yd, q, s, cols = ref.linear_decomp(X, pre, None, None, 1e-5, 6.0, Wq, s_w, G, W, bias, act)
        bc, bq, bs, bY = brute.linear_decomp(X, pre, None, None, 1e-5, 6.0, W, G, bias, act)
        assert cols.size > 0, seed
        assert np.array_equal(cols, bc) and np.array_equal(q, bq) and np.array_equal(s, bs), seed
        assert np.array_equal(Yd.view(np.uint16), bY.view(np.uint16)), seed


def pin_decomp_rows_subset():
    """The row-subset form finds O from every token and then gives exactly the
    listed rows of the full result."""
    X, W, bias, _ = _decomp_case(50, 12, 64, 8, 2, x_dtype=np.float16)
    Wq, s_w = ref.quantize_groups(W, 2)
    Yd, q, s, cols = ref.linear_decomp(X, ref.PRE_LAYERNORM, None, None, 1e-5, 6.0, Wq, s_w, 2, W,
                                       bias, ref.ACT_GELU)
    rows = np.array([11, 0, 5])
    Yr, qr, sr, cr = ref.linear_decomp_rows(X, ref.PRE_LAYERNORM, None, None, 1e-5, 6.0, Wq, s_w, 2,
                                            W, bias, ref.ACT_GELU, rows)
    assert np.array_equal(cr, cols) and cols.size > 0
    assert np.array_equal(qr, q[rows]) and np.array_equal(sr, s[rows])
    assert np.array_equal(Yr.view(np.uint16), Yd[rows].view(np.uint16))



# --------------------------------------------------------------------------
# The row-subset and unquantized forms used as references for the full-size
# workloads ("探秘Transformer系列之（36）" 1.2.2: every token is quantized with
# its own scale, so a token's output depends on that token's row alone)
# --------------------------------------------------------------------------

def pin_linear_rows_is_subset_of_linear():
    """linear_rows(rows) equals the listed rows of linear() bit for bit, for
    fp16 and fp32 X, LayerNorm (with an affine) and GeLU, rows listed out of
    order and with a repeat."""
    rng = np.random.default_rng(60)
    M, K, N, G = 11, 48, 12, 4
    rows = np.array([7, 0, 10, 3, 7, 5])
    for x_dtype in (np.float16, np.float32):
        X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(x_dtype)
        W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
        bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
        gamma = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
        beta = (0.1 * rng.standard_normal(K)).astype(np.float32)
        Wq, s_w = ref.quantize_groups(W, G)
        for pre, act, g, b in ((ref.PRE_LAYERNORM, ref.ACT_NONE, gamma, beta),
                               (ref.PRE_GELU, ref.ACT_GELU, None, None),
                               (ref.PRE_NONE, ref.ACT_GELU, None, None)):
            Y, q, s = ref.linear(X, pre, g, b, 1e-5, Wq, s_w, G, bias, act)
            Yr, qr, sr = ref.linear_rows(X, pre, g, b, 1e-5, Wq, s_w, G, bias, act, rows)
            assert np.array_equal(qr, q[rows]) and np.array_equal(sr, s[rows]), (x_dtype, pre)
            assert np.array_equal(Yr.view(np.uint16), Y[rows].view(np.uint16)), (x_dtype, pre)


def pin_linear_float_rows_is_plain_matmul():
    """The unquantized layer equals preop(X)[rows] W^T + b (+ erf GeLU)
    written with numpy's float64 matmul and scipy's erf, to 1e-12 of the sum
    of the terms' magnitudes."""
    from scipy.special import erf
    rng = np.random.default_rng(61)
    M, K, N = 9, 64, 10
    X = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    bias = (0.5 * rng.standard_normal(N)).astype(np.float32)
    rows = np.array([8, 2, 4])
    for pre, act in ((ref.PRE_LAYERNORM, ref.ACT_NONE), (ref.PRE_GELU, ref.ACT_GELU)):
        got = ref.linear_float_rows(X, pre, None, None, 1e-5, W, bias, act, rows)
        y = ref.preop(X, pre)[rows].astype(np.float64)
        v = y @ W.astype(np.float64).T + bias.astype(np.float64)
        mag = np.abs(y) @ np.abs(W.astype(np.float64)).T + np.abs(bias)
        if act == ref.ACT_GELU:
            v = 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))
        assert np.all(np.abs(got - v) <= 1e-12 * mag), pre
    # without a bias the output changes by exactly the bias
    nob = ref.linear_float_rows(X, ref.PRE_LAYERNORM, None, None, 1e-5, W, None, ref.ACT_NONE, rows)
    wib = ref.linear_float_rows(X, ref.PRE_LAYERNORM, None, None, 1e-5, W, bias, ref.ACT_NONE, rows)
    np.testing.assert_allclose(wib - nob, np.broadcast_to(bias.astype(np.float64), nob.shape),
                               rtol=0, atol=1e-12)


def pin_fp8_group_special_cases():
    """FP8 group codes: G = N is one power-of-two scale over the whole tensor
    (the per-row quantizer applied to the flattened tensor), G = 1 is the
    per-row quantizer on each row, and an intermediate G takes each block of
    G consecutive rows on its own ("探秘Transformer系列之（36）" 1.3 granularity)."""
    rng = np.random.default_rng(62)
    N, K = 12, 40
    W = (0.02 * rng.standard_normal((N, K)) * np.exp(2 * rng.standard_normal((N, 1)))).astype(np.float32)
    q, s = ref.quantize_groups_fp8(W, N)
    qt, st = ref.quantize_rows_fp8(W.reshape(1, N * K))
    assert np.array_equal(q.ravel(), qt.ravel()) and s[0] == st[0]
    q, s = ref.quantize_groups_fp8(W, 1)
    qr, sr = ref.quantize_rows_fp8(W)
    assert np.array_equal(q, qr) and np.array_equal(s, sr)
    q, s = ref.quantize_groups_fp8(W, 4)
    for g in range(3):
        qg, sg = ref.quantize_rows_fp8(W[4 * g:4 * g + 4].reshape(1, 4 * K))
        assert np.array_equal(q[4 * g:4 * g + 4].ravel(), qg.ravel()) and s[g] == sg[0], g


def pin_smoothquant_identity_fp32():
    """The SmoothQuant identity (X diag(s)^-1)(diag(s) W) = X W holds to 1e-5
    relative (max norm) with both products taken in fp32 ("SmoothQuant技术解析"
    2.2), on the oracle's fp32 factors and folded weights."""
    rng = np.random.default_rng(63)
    M, K, N = 64, 256, 96
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, [3, 100, 201]] *= np.float32(100.0)
    X = X.astype(np.float16)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    s = ref.smooth_factors(X, W)
    Xt = ref.preop(X, ref.PRE_LAYERNORM)
    Xh = (Xt / s).astype(np.float32)
    Wh = ref.fold_weights(W, s)
    Y0 = np.matmul(Xt, W.T, dtype=np.float32)
    Y1 = np.matmul(Xh, Wh.T, dtype=np.float32)
    assert Y0.dtype == np.float32 and Y1.dtype == np.float32
    assert np.max(np.abs(Y1 - Y0)) <= 1e-5 * np.max(np.abs(Y0))
    # a wrong fold (W divided instead of multiplied) is far outside it
    bad = np.matmul(Xh, (W / s).astype(np.float32).T, dtype=np.float32)
    assert np.max(np.abs(bad - Y0)) > 1e-2 * np.max(np.abs(Y0))

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
