"""Seeded synthetic inputs for the W8A8 linear layer.

This module only draws random numbers and casts them to their storage dtype.
It holds none of the method's arithmetic (no normalisation, no quantization,
no smoothing): both the HIP path and the CPU oracle receive the same arrays
from here and compute everything else themselves.

Five workloads, each shaped like a transformer linear layer that the pages
discuss (BERT / GPT / LLaMA-scale layers):

  tiny          X fp32 [16 x 256],    LayerNorm prologue, W [256 x 256],  G=64,  bias, fp16 out
  bert_ffn_up   X fp16 [4096 x 768],  LayerNorm prologue, W [3072 x 768], G=128, bias + GeLU epilogue
  gpt_qkv       X fp16 [2048 x 4096], LayerNorm prologue, W [12288 x 4096], G=128, bias
  decode_ffn_down X fp16 [16 x 28672], GeLU prologue,     W [8192 x 28672], G=128, no bias
  outlier_smooth X fp16 [4096 x 5120] with 0.5% of channels x100, LayerNorm prologue
                 with a SmoothQuant fold, W [13824 x 5120], G=128, no bias

Draw order per workload (fixed, one numpy Generator seeded with 0):
X standard normal -> per-token log-scale -> W standard normal -> per-row
log-scale -> bias -> outlier channel set.  Values are drawn in fp32 and X is
cast to its storage dtype afterwards.  W stays fp32 (it is quantized offline
by each side).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

PRE_NONE, PRE_LAYERNORM, PRE_GELU = 0, 1, 2
ACT_NONE, ACT_GELU = 0, 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    group_rows: int
    x_dtype: str            # "f32" or "f16"
    pre: int                # PRE_*
    act: int                # ACT_*
    has_bias: bool
    token_logscale: float   # sigma of the per-token lognormal scale (0 = none)
    w_std: float
    row_logscale: float     # sigma of the per-row lognormal range of W (0 = none)
    outlier_frac: float     # fraction of input channels scaled by outlier_gain
    outlier_gain: float
    smooth: bool            # fold SmoothQuant factors into LN gamma/beta and W
    eps: float = 1e-5
    seed: int = 0

    @property
    def ops(self) -> int:
        """Integer multiply-adds counted as 2 ops each: 2*M*N*K."""
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 16, 256, 256, 64, "f32", PRE_LAYERNORM, ACT_NONE, True,
                 1.0, 0.02, 0.0, 0.0, 1.0, False),
        Workload("bert_ffn_up", 4096, 768, 3072, 128, "f16", PRE_LAYERNORM, ACT_GELU, True,
                 1.0, 0.02, 0.5, 0.0, 1.0, False),
        Workload("gpt_qkv", 2048, 4096, 12288, 128, "f16", PRE_LAYERNORM, ACT_NONE, True,
                 1.0, 0.02, 0.0, 0.0, 1.0, False),
        Workload("decode_ffn_down", 16, 28672, 8192, 128, "f16", PRE_GELU, ACT_NONE, False,
                 1.0, 0.02, 0.0, 0.0, 1.0, False),
        Workload("outlier_smooth", 4096, 5120, 13824, 128, "f16", PRE_LAYERNORM, ACT_NONE, False,
                 0.0, 0.02, 0.0, 0.005, 100.0, True),
    ]
}

# The order in which the workloads are listed in the task's configuration.
WORKLOAD_ORDER = ["tiny", "bert_ffn_up", "gpt_qkv", "decode_ffn_down", "outlier_smooth"]


@dataclasses.dataclass
class Inputs:
    X: np.ndarray                 # [M, K] float32 or float16, row-major
    W: np.ndarray                 # [N, K] float32, row-major (output rows, input columns)
    bias: Optional[np.ndarray]    # [N] float32 or None
    gamma: np.ndarray             # [K] float32 (ones)
    beta: np.ndarray              # [K] float32 (zeros)
    outlier_channels: Optional[np.ndarray]  # int64 indices or None


def make_inputs(w: Workload, M: Optional[int] = None, seed: Optional[int] = None) -> Inputs:
    """Draw the workload's inputs.  `M` overrides the token count (same recipe,
    fewer or more rows); `seed` overrides the seed."""
    M = w.M if M is None else int(M)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    X = rng.standard_normal((M, w.K), dtype=np.float32)
    if w.token_logscale > 0:
        X *= np.exp(w.token_logscale * rng.standard_normal((M, 1), dtype=np.float32))
    W = rng.standard_normal((w.N, w.K), dtype=np.float32)
    W *= np.float32(w.w_std)
    if w.row_logscale > 0:
        W *= np.exp(w.row_logscale * rng.standard_normal((w.N, 1), dtype=np.float32))
    bias = None
    if w.has_bias:
        bias = (np.float32(0.01) * rng.standard_normal(w.N, dtype=np.float32)).astype(np.float32)
    outl = None
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * w.K))
        outl = np.sort(rng.choice(w.K, n_out, replace=False)).astype(np.int64)
        X[:, outl] *= np.float32(w.outlier_gain)
    X = X.astype(np.float16 if w.x_dtype == "f16" else np.float32)
    gamma = np.ones(w.K, dtype=np.float32)
    beta = np.zeros(w.K, dtype=np.float32)
    return Inputs(X=np.ascontiguousarray(X), W=np.ascontiguousarray(W), bias=bias,
                  gamma=gamma, beta=beta, outlier_channels=outl)


def random_int8(rng: np.random.Generator, shape, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Uniform int8 codes in [lo, hi] (used to drive the integer GEMM on its own)."""
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int8)


def random_affine(rng: np.random.Generator, K: int):
    """LayerNorm gamma ~ 1 + 0.1 N(0,1), beta ~ 0.1 N(0,1) for tests that vary them."""
    g = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    b = (0.1 * rng.standard_normal(K)).astype(np.float32)
    return g, b
