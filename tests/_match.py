"""Matching rules between the HIP path and the CPU oracle.

- int32 accumulators, weight codes and weight scales: bit-exact.
- Activation codes: |diff| <= 1 everywhere and |diff| == 1 on at most
  floor(1e-4 n) of the n elements (none at all below 10^4 elements).
  LayerNorm reductions run in a different order (fp32 on the GPU, fp64 in
  the oracle), so a value that lands within rounding of a half-integer may
  round either way; nothing else may differ.
- Per-token scales: within 4 fp32 ulps.
- fp16 outputs: max |dY| <= 1e-2 * max |Y_ref| and normwise mean relative
  error sum |dY| / sum |Y_ref| <= 1e-3.
- FP8 (E4M3) activation codes: the same byte, or the neighbouring code of the
  same sign, on at most max(1, 1e-4 n) elements.
"""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def assert_codes(got: np.ndarray, want: np.ndarray, what: str = "codes", exact: bool = False):
    got = np.asarray(got).astype(np.int32)
    want = np.asarray(want).astype(np.int32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    d = np.abs(got - want)
    if exact:
        assert d.max(initial=0) == 0, f"{what}: {int((d > 0).sum())} codes differ"
        return 0
    assert d.max(initial=0) <= 1, f"{what}: max code difference {d.max()}"
    flips = int((d == 1).sum())
    allowed = int(1e-4 * d.size)
    if flips:
        say(f"{what}: {flips} +-1 flips of {d.size} ({allowed} allowed)")
    assert flips <= allowed, f"{what}: {flips} +-1 flips > {allowed} allowed of {d.size}"
    return flips


def assert_scales(got: np.ndarray, want: np.ndarray, what: str = "scales", ulps: int = 4):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    tol = ulps * np.spacing(np.abs(want))
    d = np.abs(got.astype(np.float64) - want.astype(np.float64))
    worst = (d / np.maximum(np.spacing(np.abs(want)), 1e-45)).max(initial=0.0)
    if worst > 1:
        say(f"{what}: worst scale {worst:.1f} ulps")
    assert np.all(d <= tol), f"{what}: max diff {worst:.1f} ulps"


def y_errors(got: np.ndarray, want: np.ndarray):
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert np.all(np.isfinite(g)), "non-finite output"
    d = np.abs(g - w)
    max_rel = d.max() / max(np.abs(w).max(), 1e-30)
    mean_rel = d.sum() / max(np.abs(w).sum(), 1e-30)
    return max_rel, mean_rel


def assert_y(got: np.ndarray, want: np.ndarray, what: str = "Y"):
    max_rel, mean_rel = y_errors(got, want)
    assert max_rel <= 1e-2, f"{what}: max |dY| / max |Y| = {max_rel:.3e}"
    assert mean_rel <= 1e-3, f"{what}: sum |dY| / sum |Y| = {mean_rel:.3e}"
    return max_rel, mean_rel


def assert_fp8_codes(got, want):
    """Same byte, or the neighbouring code of the same sign (a near-tie decided
    on a value one fp32 ulp away), on at most max(1, 1e-4 n) elements."""
    g = np.asarray(got).astype(np.int16)
    w = np.asarray(want).astype(np.int16)
    off = g != w
    same_sign = (g & 0x80) == (w & 0x80)
    assert np.all(np.abs(g - w)[off] <= 1) and np.all(same_sign[off]), "codes differ by more than one step"
    assert off.sum() <= max(1, int(1e-4 * g.size)), f"{off.sum()} codes differ"
