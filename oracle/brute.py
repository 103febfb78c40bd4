"""Pure-Python brute force of the W8A8 linear layer, for tiny shapes only.

TEST INFRASTRUCTURE ONLY.  A second CPU implementation, written separately
from oracle/zq_ref.c, used to pin it: exact sums with math.fsum, Python
integers for the GEMM, numpy's own float16 rounding for the output.  The
two must agree bit for bit on codes, scales and accumulators.

Pages: "Integer Quantization: Deep Dive" ("如何进行量化？", z = 0);
"探秘Transformer系列之（36）--- 大模型量化方案" 1.1.2 (absmax to [-127, 127]),
1.2.2 (per-token activations, group-wise weights, INT32 accumulation scaled
before the FP16 write); ZeroQuant reading notes (fused LN/GeLU + Quantize).
"""
from __future__ import annotations

import math

import numpy as np

PRE_NONE, PRE_LAYERNORM, PRE_GELU = 0, 1, 2
ACT_NONE, ACT_GELU = 0, 1


def _f32(v: float) -> float:
    return float(np.float32(v))


def preop_row(x, pre, gamma=None, beta=None, eps=1e-5):
    xs = [float(v) for v in x]
    K = len(xs)
    if pre == PRE_LAYERNORM:
        mu = math.fsum(xs) / K
        var = math.fsum((v - mu) ** 2 for v in xs) / K
        r = 1.0 / math.sqrt(var + float(np.float32(eps)))
        g = [1.0] * K if gamma is None else [float(v) for v in gamma]
        b = [0.0] * K if beta is None else [float(v) for v in beta]
        return [_f32((xs[k] - mu) * r * g[k] + b[k]) for k in range(K)]
    if pre == PRE_GELU:
        return [_f32(0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))) for v in xs]
    return [_f32(v) for v in xs]


def quantize_vec(y):
    """absmax: s = fl32(a/127); q = clamp(round_half_even(fl32(y/s)), +-127)."""
    a = max(abs(v) for v in y)
    s = np.float32(a) / np.float32(127.0)
    if s == 0:
        return [0] * len(y), float(s)
    q = []
    for v in y:
        t = float(np.float32(v) / s)
        r = round(t)                # Python rounds halves to even
        q.append(max(-127, min(127, r)))
    return q, float(s)


def linear(X, pre, gamma, beta, eps, W, G, bias, act):
    """Returns (Xq, s_x, Wq, s_w, acc, Y_fp16) as Python lists / numpy arrays."""
    X = np.asarray(X)
    W = np.asarray(W, dtype=np.float32)
    M, K = X.shape
    N = W.shape[0]
    Xq, s_x = [], []
    for m in range(M):
        q, s = quantize_vec(preop_row(X[m].astype(np.float64), pre, gamma, beta, eps))
        Xq.append(q)
        s_x.append(s)
    Wq, s_w = [None] * N, []
    for g in range(N // G):
        flat = [float(v) for v in W[g * G:(g + 1) * G].ravel()]
        q, s = quantize_vec(flat)
        s_w.append(s)
        for i in range(G):
            Wq[g * G + i] = q[i * K:(i + 1) * K]
    acc = [[sum(Xq[m][k] * Wq[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    Y = np.empty((M, N), dtype=np.float16)
    for m in range(M):
        for n in range(N):
            v = s_x[m] * s_w[n // G] * acc[m][n]
            if bias is not None:
                v += float(bias[n])
            if act == ACT_GELU:
                v = 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))
            Y[m, n] = np.float16(v)     # numpy rounds float64 -> float16 once, ties to even
    return (np.array(Xq, dtype=np.int8), np.array(s_x, dtype=np.float32),
            np.array(Wq, dtype=np.int8), np.array(s_w, dtype=np.float32),
            np.array(acc, dtype=np.int64), Y)


def linear_decomp(X, pre, gamma, beta, eps, alpha, W, G, bias, act):
    """LLM.int8() mixed-precision decomposition ("探秘Transformer系列之（36）" 1.1,
    "方案" and "混合精度分解"), written separately from the C oracle:
    outlier columns are those where some |y| exceeds alpha; they are taken in
    FP16 on both sides; the rest are absmax-quantized per token and per weight
    group; the two partial products are summed exactly (math.fsum) and
    rounded to fp16 once.  Returns (cols, Xq, s_x, Y_fp16)."""
    X = np.asarray(X)
    W = np.asarray(W, dtype=np.float32)
    M, K = X.shape
    N = W.shape[0]
    rows = [preop_row(X[m].astype(np.float64), pre, gamma, beta, eps) for m in range(M)]
    cols = [j for j in range(K) if any(abs(rows[m][j]) > alpha for m in range(M))]
    outl = set(cols)
    Xq, s_x = [], []
    for m in range(M):
        keep = [rows[m][j] if j not in outl else 0.0 for j in range(K)]
        q, s = quantize_vec(keep)
        Xq.append(q)
        s_x.append(s)
    Wq, s_w = [None] * N, []
    for g in range(N // G):
        q, s = quantize_vec([float(v) for v in W[g * G:(g + 1) * G].ravel()])
        s_w.append(s)
        for i in range(G):
            Wq[g * G + i] = q[i * K:(i + 1) * K]
    h = lambda v: float(np.float16(v))      # numpy's own nearest-even fp16 rounding
    Y = np.empty((M, N), dtype=np.float16)
    for m in range(M):
        for n in range(N):
            acc = sum(Xq[m][k] * Wq[n][k] for k in range(K))
            terms = [s_x[m] * s_w[n // G] * acc]
            terms += [h(rows[m][j]) * h(W[n, j]) for j in cols]
            if bias is not None:
                terms.append(float(bias[n]))
            v = math.fsum(terms)
            if act == ACT_GELU:
                v = 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))
            Y[m, n] = np.float16(v)
    return (np.array(cols, dtype=np.int32), np.array(Xq, dtype=np.int8),
            np.array(s_x, dtype=np.float32), Y)
