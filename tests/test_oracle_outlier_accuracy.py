"""Accuracy of the two outlier treatments on the outlier workload, from the
oracle alone (CPU): the layer's output on sampled tokens against the
unquantized layer in fp64.

The pages present SmoothQuant's per-channel smoothing and LLM.int8()'s
mixed-precision decomposition as two answers to activation outliers that
ruin a per-token int8 scale ("探秘Transformer系列之（36）--- 大模型量化方案" 1.1
and the comparison that follows ZeroQuant; "SmoothQuant技术解析" 2.2).  The
checked property: both treatments are more accurate than plain W8A8 on
inputs with outlier channels.  The figures are printed for the record.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

from oracle import ref
from zq_workloads import WORKLOADS, make_inputs


def _err(Y, Yf):
    Y = np.asarray(Y, dtype=np.float64)
    return np.abs(Y - Yf).sum() / np.abs(Yf).sum(), np.abs(Y - Yf).max() / np.abs(Yf).max()


@pytest.mark.timeout(600)
def test_outlier_treatments_beat_plain_w8a8():
    w = WORKLOADS["outlier_smooth"]
    inp = make_inputs(w)
    X, W = inp.X, inp.W
    rows = np.linspace(0, w.M - 1, 12).astype(np.int64)
    pre, eps = w.pre, w.eps
    Yf = ref.linear_float_rows(X, pre, None, None, eps, W, None, w.act, rows)

    Wq, s_w = ref.quantize_groups(W, 128)
    Y_plain = ref.linear_rows(X, pre, None, None, eps, Wq, s_w, 128, None, w.act, rows)[0]

    s = ref.smooth_factors(X, W, eps)
    g, b = ref.fold_ln(None, None, s)
    Wsq, s_ws = ref.quantize_groups(ref.fold_weights(W, s), 128)
    Y_smooth = ref.linear_rows(X, pre, g, b, eps, Wsq, s_ws, 128, None, w.act, rows)[0]

    out = {}
    for G in (1, 128):
        Wq_g, s_w_g = (Wq, s_w) if G == 128 else ref.quantize_groups(W, G)
        Yd, _, _, cols = ref.linear_decomp_rows(X, pre, None, None, eps, 6.0, Wq_g, s_w_g, G, W,
                                                None, w.act, rows)
        assert np.array_equal(cols, inp.outlier_channels)
        out[G] = _err(Yd, Yf)

    e_plain, e_smooth = _err(Y_plain, Yf), _err(Y_smooth, Yf)
    print(f"[outlier workload, {rows.size} tokens] sum|dY|/sum|Y| (max|dY|/max|Y|): "
          f"plain W8A8 G=128 {e_plain[0]:.3e} ({e_plain[1]:.3e}); "
          f"SmoothQuant G=128 {e_smooth[0]:.3e} ({e_smooth[1]:.3e}); "
          f"decomposition G=1 {out[1][0]:.3e} ({out[1][1]:.3e}); "
          f"decomposition G=128 {out[128][0]:.3e} ({out[128][1]:.3e})", file=sys.stderr)
    assert e_smooth[0] < e_plain[0]
    assert out[1][0] < e_plain[0] and out[128][0] < e_plain[0]
