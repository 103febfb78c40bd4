"""NumPy-facing wrapper of the CPU oracle (oracle/zq_ref.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg call this; the HIP library never does.
Every function takes and returns host numpy arrays and states the page
passage it follows in the C source it wraps.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzqref.so")

PRE_NONE, PRE_LAYERNORM, PRE_GELU = 0, 1, 2
ACT_NONE, ACT_GELU = 0, 1

_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_f = ctypes.c_float

_SIGS = {
    "zqref_set_threads": (None, [_i]),
    "zqref_max_threads": (_i, []),
    "zqref_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "zqref_f64_to_f16": (ctypes.c_uint16, [ctypes.c_double]),
    "zqref_preop": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _p]),
    "zqref_quantize_rows": (_i, [_p, _i64, _i64, _p, _p]),
    "zqref_round_to_f16": (_i, [_p, _i64, _p]),
    "zqref_e4m3_to_f64": (ctypes.c_double, [ctypes.c_uint8]),
    "zqref_f64_to_e4m3": (ctypes.c_uint8, [ctypes.c_double]),
    "zqref_pow2_scale": (ctypes.c_float, [ctypes.c_float]),
    "zqref_quantize_rows_fp8": (_i, [_p, _i64, _i64, _p, _p]),
    "zqref_quantize_groups_fp8": (_i, [_p, _i64, _i64, _i64, _p, _p]),
    "zqref_gemm_fp8": (_i, [_p, _p, _i64, _i64, _i64, _p]),
    "zqref_epilogue_f64acc": (_i, [_p, _p, _p, _i64, _p, _i, _i64, _i64, _p]),
    "zqref_prologue": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _p, _p, _p]),
    "zqref_quantize_groups": (_i, [_p, _i64, _i64, _i64, _p, _p]),
    "zqref_smooth_factors": (_i, [_p, _i, _i64, _i64, _f, _p, _i64, _p]),
    "zqref_fold_ln": (_i, [_p, _p, _p, _i64, _p, _p]),
    "zqref_fold_weights": (_i, [_p, _p, _i64, _i64, _p]),
    "zqref_gemm_i32": (_i, [_p, _p, _i64, _i64, _i64, _p]),
    "zqref_epilogue": (_i, [_p, _p, _p, _i64, _p, _i, _i64, _i64, _p, _p]),
    "zqref_linear_rows": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _p, _p, _i64, _p, _i,
                               _i64, _p, _i64, _p, _p, _p]),
    "zqref_linear_float_rows": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _p, _p, _i, _i64,
                                     _p, _i64, _p]),
    "zqref_outlier_columns": (_i, [_p, _i64, _i64, _f, _p, _p]),
    "zqref_quantize_rows_excluding": (_i, [_p, _i64, _i64, _p, _i64, _p, _p]),
    "zqref_decomp_epilogue": (_i, [_p, _p, _p, _i64, _p, _i64, _p, _i64, _p, _p, _i, _i64, _i64,
                                   _p, _p]),
    "zqref_linear_decomp_rows": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _f, _p, _p, _i64, _p,
                                      _p, _i, _i64, _p, _i64, _p, _p, _p, _p, _p]),
}


class OracleError(RuntimeError):
    pass


def _load(path: str):
    L = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """Load the compiled oracle, building it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b
            _b.build()
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every wrapper through another build of the oracle
    (the mutation tests use this to check that the pins catch planted bugs)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def set_threads(n: int) -> None:
    """Thread count of the oracle's parallel loops (timing only; results do not depend on it)."""
    lib().zqref_set_threads(int(n))


def max_threads() -> int:
    return int(lib().zqref_max_threads())


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def _x_args(X: np.ndarray):
    if X.dtype == np.float16:
        return 1
    if X.dtype == np.float32:
        return 0
    raise TypeError(f"X must be float16 or float32, got {X.dtype}")


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    L = lib()
    h = np.asarray(h, dtype=np.uint16).ravel()
    return np.array([L.zqref_f16_to_f32(int(v)) for v in h], dtype=np.float32)


def f64_to_f16_bits(v: Sequence[float]) -> np.ndarray:
    L = lib()
    return np.array([L.zqref_f64_to_f16(float(x)) for x in v], dtype=np.uint16)


def preop(X: np.ndarray, pre: int, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """y = LN(x) / GeLU(x) / x in the oracle's precision, rounded once to fp32."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    Y = np.empty((M, K), dtype=np.float32)
    _check(lib().zqref_preop(_ptr(X), _x_args(X), M, K, pre, _ptr(gamma), _ptr(beta), eps, _ptr(Y)),
           "zqref_preop")
    return Y


def quantize_rows(Y: np.ndarray):
    """Dynamic per-row absmax quantization of fp32 rows -> (int8 codes, fp32 scales)."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    M, K = Y.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    _check(lib().zqref_quantize_rows(_ptr(Y), M, K, _ptr(q), _ptr(s)), "zqref_quantize_rows")
    return q, s


def round_to_f16(Y: np.ndarray) -> np.ndarray:
    """fp32 values rounded once to binary16 (nearest even) and widened back to fp32."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    out = np.empty_like(Y)
    _check(lib().zqref_round_to_f16(_ptr(Y), Y.size, _ptr(out)), "zqref_round_to_f16")
    return out


def unfused_prologue(X: np.ndarray, pre: int, gamma=None, beta=None, eps: float = 1e-5):
    """The unfused order (ZeroQuant reading notes, kernel-fusion figure before fusion):
    LN/GeLU -> FP16 tensor in memory -> separate per-token quantization.
    Returns (Xq int8 [M,K], s_x fp32 [M])."""
    return quantize_rows(round_to_f16(preop(X, pre, gamma, beta, eps)))


# ---- FP8 variant (ZeroQuant-FP: FP8 E4M3 codes, power-of-two scales) ----

def e4m3_to_f64(codes) -> np.ndarray:
    L = lib()
    return np.array([L.zqref_e4m3_to_f64(int(c)) for c in np.asarray(codes, np.uint8).ravel()])


def f64_to_e4m3(v) -> np.ndarray:
    L = lib()
    return np.array([L.zqref_f64_to_e4m3(float(x)) for x in np.asarray(v).ravel()], np.uint8)


def pow2_scale(a: float) -> float:
    return float(lib().zqref_pow2_scale(float(np.float32(a))))


def quantize_rows_fp8(Y: np.ndarray):
    """Per-row FP8 E4M3 codes with power-of-two scales -> (uint8 codes, fp32 scales)."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    M, K = Y.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty(M, dtype=np.float32)
    _check(lib().zqref_quantize_rows_fp8(_ptr(Y), M, K, _ptr(q), _ptr(s)), "zqref_quantize_rows_fp8")
    return q, s


def prologue_fp8(X: np.ndarray, pre: int, gamma=None, beta=None, eps: float = 1e-5):
    """LN/GeLU in fp32 then per-token FP8 codes with power-of-two scales."""
    return quantize_rows_fp8(preop(X, pre, gamma, beta, eps))


def quantize_groups_fp8(W: np.ndarray, G: int):
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(N // G, dtype=np.float32)
    _check(lib().zqref_quantize_groups_fp8(_ptr(W), N, K, G, _ptr(q), _ptr(s)),
           "zqref_quantize_groups_fp8")
    return q, s


def gemm_fp8(Xq: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """acc = dec(Xq) dec(Wq)^T summed in fp64."""
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    M, K = Xq.shape
    N = Wq.shape[0]
    acc = np.empty((M, N), dtype=np.float64)
    _check(lib().zqref_gemm_fp8(_ptr(Xq), _ptr(Wq), M, N, K, _ptr(acc)), "zqref_gemm_fp8")
    return acc


def epilogue_f64acc(acc: np.ndarray, s_x, s_w, G: int, bias=None, act: int = ACT_NONE):
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    M, N = acc.shape
    Y = np.empty((M, N), dtype=np.uint16)
    _check(lib().zqref_epilogue_f64acc(_ptr(acc), _ptr(np.ascontiguousarray(s_x, np.float32)),
                                       _ptr(np.ascontiguousarray(s_w, np.float32)), G,
                                       _ptr(None if bias is None else np.ascontiguousarray(bias, np.float32)),
                                       act, M, N, _ptr(Y)), "zqref_epilogue_f64acc")
    return Y.view(np.float16)


def linear_fp8(X, pre, gamma, beta, eps, Wq8, s_w, G, bias, act):
    """The FP8 layer on all tokens -> (Y fp16, codes, scales)."""
    q, s = prologue_fp8(X, pre, gamma, beta, eps)
    return epilogue_f64acc(gemm_fp8(q, Wq8), s, s_w, G, bias, act), q, s


def prologue(X: np.ndarray, pre: int, gamma=None, beta=None, eps: float = 1e-5,
             return_y: bool = False):
    """Fused LN/GeLU + per-token quantization -> (Xq int8 [M,K], s_x fp32 [M])."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    Y = np.empty((M, K), dtype=np.float32) if return_y else None
    _check(lib().zqref_prologue(_ptr(X), _x_args(X), M, K, pre, _ptr(gamma), _ptr(beta), eps,
                                _ptr(q), _ptr(s), _ptr(Y)), "zqref_prologue")
    return (q, s, Y) if return_y else (q, s)


def quantize_groups(W: np.ndarray, G: int):
    """Group-wise weight quantization, G consecutive output rows per group."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    q = np.empty((N, K), dtype=np.int8)
    s = np.empty(N // G, dtype=np.float32)
    _check(lib().zqref_quantize_groups(_ptr(W), N, K, G, _ptr(q), _ptr(s)), "zqref_quantize_groups")
    return q, s


def smooth_factors(X: np.ndarray, W: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    X = np.ascontiguousarray(X)
    W = np.ascontiguousarray(W, dtype=np.float32)
    M, K = X.shape
    N = W.shape[0]
    s = np.empty(K, dtype=np.float32)
    _check(lib().zqref_smooth_factors(_ptr(X), _x_args(X), M, K, eps, _ptr(W), N, _ptr(s)),
           "zqref_smooth_factors")
    return s


def fold_ln(gamma, beta, s: np.ndarray):
    K = s.shape[0]
    g = np.empty(K, dtype=np.float32)
    b = np.empty(K, dtype=np.float32)
    _check(lib().zqref_fold_ln(_ptr(gamma), _ptr(beta), _ptr(s), K, _ptr(g), _ptr(b)), "zqref_fold_ln")
    return g, b


def fold_weights(W: np.ndarray, s: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    out = np.empty((N, K), dtype=np.float32)
    _check(lib().zqref_fold_weights(_ptr(W), _ptr(s), N, K, _ptr(out)), "zqref_fold_weights")
    return out


def gemm_i32(Xq: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """acc[m,n] = sum_k Xq[m,k] * Wq[n,k], exact."""
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    M, K = Xq.shape
    N = Wq.shape[0]
    acc = np.empty((M, N), dtype=np.int32)
    _check(lib().zqref_gemm_i32(_ptr(Xq), _ptr(Wq), M, N, K, _ptr(acc)), "zqref_gemm_i32")
    return acc


def epilogue(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray, G: int, bias=None,
             act: int = ACT_NONE, return_f64: bool = False):
    """Dequant + bias (+GeLU) -> fp16 (returned as np.float16)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    M, N = acc.shape
    Y = np.empty((M, N), dtype=np.uint16)
    Y64 = np.empty((M, N), dtype=np.float64) if return_f64 else None
    _check(lib().zqref_epilogue(_ptr(acc), _ptr(np.ascontiguousarray(s_x, np.float32)),
                                _ptr(np.ascontiguousarray(s_w, np.float32)), G, _ptr(bias), act,
                                M, N, _ptr(Y), _ptr(Y64)), "zqref_epilogue")
    Yh = Y.view(np.float16)
    return (Yh, Y64) if return_f64 else Yh


def linear(X, pre, gamma, beta, eps, Wq, s_w, G, bias, act):
    """The whole layer on all tokens: prologue -> exact int GEMM -> epilogue."""
    Xq, s_x = prologue(X, pre, gamma, beta, eps)
    acc = gemm_i32(Xq, Wq)
    return epilogue(acc, s_x, s_w, G, bias, act), Xq, s_x


def linear_rows(X, pre, gamma, beta, eps, Wq, s_w, G, bias, act, rows):
    """The whole layer evaluated only for the tokens in `rows`."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    N = Wq.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.shape[0]
    Xq = np.empty((R, K), dtype=np.int8)
    s_x = np.empty(R, dtype=np.float32)
    Y = np.empty((R, N), dtype=np.uint16)
    _check(lib().zqref_linear_rows(_ptr(X), _x_args(X), M, K, pre, _ptr(gamma), _ptr(beta), eps,
                                   _ptr(np.ascontiguousarray(Wq, np.int8)),
                                   _ptr(np.ascontiguousarray(s_w, np.float32)), G, _ptr(bias), act,
                                   N, _ptr(rows), R, _ptr(Xq), _ptr(s_x), _ptr(Y)),
           "zqref_linear_rows")
    return Y.view(np.float16), Xq, s_x


def linear_float_rows(X, pre, gamma, beta, eps, W, bias, act, rows):
    """Unquantized act(preop(X) W^T + b) in fp64 for the tokens in `rows`."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    W = np.ascontiguousarray(W, dtype=np.float32)
    N = W.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    Y = np.empty((rows.shape[0], N), dtype=np.float64)
    _check(lib().zqref_linear_float_rows(_ptr(X), _x_args(X), M, K, pre, _ptr(gamma), _ptr(beta),
                                         eps, _ptr(W), _ptr(bias), act, N, _ptr(rows),
                                         rows.shape[0], _ptr(Y)), "zqref_linear_float_rows")
    return Y


# ---- LLM.int8() mixed-precision decomposition (outlier columns in FP16) ----

def outlier_columns(Y: np.ndarray, alpha: float) -> np.ndarray:
    """Ascending int32 indices j with max_m |Y[m, j]| > alpha."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    M, K = Y.shape
    cols = np.empty(K, dtype=np.int32)
    P = ctypes.c_int64(0)
    _check(lib().zqref_outlier_columns(_ptr(Y), M, K, alpha, _ptr(cols), ctypes.byref(P)),
           "zqref_outlier_columns")
    return cols[:P.value].copy()


def quantize_rows_excluding(Y: np.ndarray, cols: np.ndarray):
    """Per-row absmax quantization over the columns outside `cols`; code 0 in
    those columns -> (int8 codes, fp32 scales)."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    M, K = Y.shape
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    _check(lib().zqref_quantize_rows_excluding(_ptr(Y), M, K, _ptr(cols), cols.shape[0], _ptr(q),
                                               _ptr(s)), "zqref_quantize_rows_excluding")
    return q, s


def decomp_epilogue(acc, s_x, s_w, G: int, Y, cols, W, bias=None, act: int = ACT_NONE,
                    return_f64: bool = False):
    """Dequantized INT8 part + FP16 outlier part + bias (+GeLU) -> fp16."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    M, N = acc.shape
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.float32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    K = Y.shape[1]
    out = np.empty((M, N), dtype=np.uint16)
    out64 = np.empty((M, N), dtype=np.float64) if return_f64 else None
    _check(lib().zqref_decomp_epilogue(_ptr(acc), _ptr(np.ascontiguousarray(s_x, np.float32)),
                                       _ptr(np.ascontiguousarray(s_w, np.float32)), G, _ptr(Y), K,
                                       _ptr(cols), cols.shape[0], _ptr(W), _ptr(bias), act, M, N,
                                       _ptr(out), _ptr(out64)), "zqref_decomp_epilogue")
    Yh = out.view(np.float16)
    return (Yh, out64) if return_f64 else Yh


def linear_decomp(X, pre, gamma, beta, eps, alpha, Wq, s_w, G, W, bias, act,
                  return_f64: bool = False):
    """The decomposed layer on all tokens -> (Y fp16, codes, scales, outlier columns)."""
    Y = preop(X, pre, gamma, beta, eps)
    cols = outlier_columns(Y, alpha)
    Xq, s_x = quantize_rows_excluding(Y, cols)
    out = decomp_epilogue(gemm_i32(Xq, Wq), s_x, s_w, G, Y, cols, W, bias, act, return_f64)
    return out, Xq, s_x, cols


def linear_decomp_rows(X, pre, gamma, beta, eps, alpha, Wq, s_w, G, W, bias, act, rows):
    """The decomposed layer for the tokens in `rows` (the outlier set still
    comes from every token) -> (Y fp16 [R,N], codes [R,K], scales [R], columns)."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    N = Wq.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.shape[0]
    cols = np.empty(K, dtype=np.int32)
    P = ctypes.c_int64(0)
    Xq = np.empty((R, K), dtype=np.int8)
    s_x = np.empty(R, dtype=np.float32)
    Y = np.empty((R, N), dtype=np.uint16)
    _check(lib().zqref_linear_decomp_rows(
        _ptr(X), _x_args(X), M, K, pre, _ptr(gamma), _ptr(beta), eps, alpha,
        _ptr(np.ascontiguousarray(Wq, np.int8)), _ptr(np.ascontiguousarray(s_w, np.float32)), G,
        _ptr(np.ascontiguousarray(W, np.float32)), _ptr(bias), act, N, _ptr(rows), R, _ptr(cols),
        ctypes.byref(P), _ptr(Xq), _ptr(s_x), _ptr(Y)), "zqref_linear_decomp_rows")
    return Y.view(np.float16), Xq, s_x, cols[:P.value].copy()
