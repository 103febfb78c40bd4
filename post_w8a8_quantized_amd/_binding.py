"""ctypes marshalling for libzq.so.  No arithmetic of the method happens here."""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch  # imported first: libzq then binds to the HIP runtime torch already loaded

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libzq.so")
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "zq.h")

# zq.h enums
ZQ_OK = 0
_STATUS = {0: "ZQ_OK", 1: "ZQ_ERR_NULL", 2: "ZQ_ERR_SHAPE", 3: "ZQ_ERR_ALIGN", 4: "ZQ_ERR_DTYPE",
           5: "ZQ_ERR_WORKSPACE", 6: "ZQ_ERR_HIP", 7: "ZQ_ERR_UNSUPPORTED"}
F32, F16, I8, I32 = 0, 1, 2, 3
PRE_NONE, PRE_LAYERNORM, PRE_GELU = 0, 1, 2
ACT_NONE, ACT_GELU = 0, 1
PATH_AUTO, PATH_TILED, PATH_SKINNY = 0, 1, 2


class ZQError(RuntimeError):
    def __init__(self, call: str, status: int, msg: str = ""):
        self.status = status
        super().__init__(f"{call} failed: {_STATUS.get(status, status)} {msg}".rstrip())


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_SIGS = {
    "zq_quantize_weights_grouped": (_i, [_p, _i, _p, _i64, _i64, _i64, _p, _p, _p]),
    "zq_ln_quant_per_token": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _p, _p, _p]),
    "zq_w8a8_gemm_dequant": (_i, [_p, _p, _p, _p, _i64, _p, _i, _i64, _i64, _i64, _p, _i, _p]),
    "zq_w8a8_gemm_dequant_ex": (_i, [_p, _p, _p, _p, _i64, _p, _i, _i64, _i64, _i64, _p, _i, _i, _p]),
    "zq_linear_w8a8": (_i, [_p, _i, _i, _p, _p, _f, _p, _p, _i64, _p, _i, _i64, _i64, _i64, _p, _sz,
                           _p, _p]),
    "zq_linear_workspace_bytes": (_sz, [_i64, _i64]),
    "zq_linear_w8a8_noalloc": (_i, [_p, _i, _i, _p, _p, _f, _p, _p, _i64, _p, _i, _i64, _i64, _i64,
                                    _p, _p]),
    "zq_smoothquant_factors": (_i, [_p, _i, _i64, _i64, _f, _p, _i, _i64, _p, _p, _p, _p, _p, _p,
                                   _sz, _p]),
    "zq_smoothquant_workspace_bytes": (_sz, [_i64, _i64]),
    "zq_status_str": (ctypes.c_char_p, [_i]),
    "zq_packed_weights_bytes": (_sz, [_i64, _i64]),
    "zq_linear_w8a8_unfused": (_i, [_p, _i, _i, _p, _p, _f, _p, _p, _i64, _p, _i, _i64, _i64, _i64,
                                    _p, _sz, _p, _p]),
    "zq_linear_unfused_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "zq_ffn_w8a8": (_i, [_p, _i, _p, _p, _f, _p, _p, _i64, _p, _p, _p, _i64, _p, _i64, _i64, _i64,
                         _p, _sz, _p, _p]),
    "zq_ffn_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "zq_quantize_weights_grouped_fp8": (_i, [_p, _i, _p, _i64, _i64, _i64, _p, _p, _p]),
    "zq_ln_quant_per_token_fp8": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _p, _p, _p]),
    "zq_fp8_gemm_dequant": (_i, [_p, _p, _p, _p, _i64, _p, _i, _i64, _i64, _i64, _p, _i, _p]),
    "zq_linear_w8a8_fp8": (_i, [_p, _i, _i, _p, _p, _f, _p, _p, _i64, _p, _i, _i64, _i64, _i64,
                                _p, _sz, _p, _p]),
    "zq_linear_w8a8_fp8_packed": (_i, [_p, _i, _i, _p, _p, _f, _p, _p, _i64, _p, _i, _i64, _i64,
                                       _i64, _p, _sz, _p, _p]),
    "zq_pack_weights": (_i, [_p, _i64, _i64, _p, _p]),
    "zq_pack_outlier_weights": (_i, [_p, _i, _i64, _i64, _p, _p]),
    "zq_outlier_columns": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _f, _p, _p, _p]),
    "zq_ln_quant_decomp": (_i, [_p, _i, _i64, _i64, _i, _p, _p, _f, _p, _p, _p, _p, _p]),
    "zq_w8a8_gemm_decomp": (_i, [_p, _p, _p, _p, _i64, _p, _p, _p, _p, _i, _i64, _i64, _i64, _p,
                                 _p]),
    "zq_linear_w8a8_decomp": (_i, [_p, _i, _i, _p, _p, _f, _f, _p, _p, _i64, _p, _p, _i, _i64,
                                   _i64, _i64, _p, _sz, _p, _p]),
    "zq_linear_decomp_workspace_bytes": (_sz, [_i64, _i64]),
    "zq_w8a8_gemm_dequant_packed": (_i, [_p, _p, _p, _p, _i64, _p, _i, _i64, _i64, _i64, _p, _i,
                                         _p]),
    "zq_linear_w8a8_packed": (_i, [_p, _i, _i, _p, _p, _f, _p, _p, _i64, _p, _i, _i64, _i64, _i64,
                                   _p, _sz, _p, _p]),
}

_lib = None


def library_path() -> str:
    return _LIB_PATH


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()
    return {os.path.realpath(p) for p in paths if p.startswith("/")}


def library():
    """Load libzq.so (raises if it is not built).  Torch is imported before the
    library so both share torch's HIP runtime; loading a second runtime into
    the process would make torch's device pointers and streams meaningless to
    libzq, so that case raises too."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ZQError("load", 7, f"{_LIB_PATH} is not built; run "
                          "`python -m post_w8a8_quantized_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        runtimes = _hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise ZQError("load", 6, f"more than one HIP runtime mapped: {sorted(runtimes)}")
        _lib = L
    return _lib


def exported_symbols():
    """Names of the entry points zq.h declares."""
    text = open(_HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^\s*(?:zq_status|size_t|const char \*)\s*(zq_\w+)\s*\(", text,
                                 re.M)))


def _call(name: str, *args):
    st = getattr(library(), name)(*args)
    if st != ZQ_OK:
        raise ZQError(name, st)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtypes, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_ws(ws: torch.Tensor, need: int, device):
    """A caller-provided workspace: a contiguous GPU tensor on `device` holding
    at least `need` bytes (the C ABI sees only a pointer and a byte count, so a
    host tensor or a short buffer has to be caught here)."""
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.device.type != "cuda" or ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    have = ws.numel() * ws.element_size()
    if have < need:
        raise ValueError(f"workspace holds {have} bytes, {need} needed")


def _fdtype(t: torch.Tensor) -> int:
    return F16 if t.dtype == torch.float16 else F32


def quantize_weights_grouped(W: torch.Tensor, group_rows: int, smooth: Optional[torch.Tensor] = None,
                             out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Offline group-wise int8 quantization of W [N, K] (optionally W * diag(smooth)).
    Returns (Wq int8 [N, K], w_scales fp32 [N / group_rows])."""
    _need(W, "W", (torch.float32, torch.float16))
    N, K = W.shape
    if smooth is not None:
        _need(smooth, "smooth", (torch.float32,), (K,), W.device)
    if out is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
        s_w = torch.empty((max(N // group_rows, 1),), dtype=torch.float32, device=W.device)
    else:
        Wq, s_w = out
        _need(Wq, "Wq", (torch.int8,), (N, K), W.device)
        _need(s_w, "w_scales", (torch.float32,), (max(N // group_rows, 1),), W.device)
    _call("zq_quantize_weights_grouped", _ptr(W), _fdtype(W), _ptr(smooth), N, K, group_rows,
          _ptr(Wq), _ptr(s_w), _stream(W))
    return Wq, s_w


def ln_quant_per_token(X: torch.Tensor, pre: int = PRE_LAYERNORM, gamma=None, beta=None,
                       eps: float = 1e-5, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Fused LN/GeLU + per-token quantization of X [M, K] -> (Xq int8 [M, K], s_x fp32 [M])."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if out is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
        s_x = torch.empty((M,), dtype=torch.float32, device=X.device)
    else:
        Xq, s_x = out
        _need(Xq, "Xq", (torch.int8,), (M, K), X.device)
        _need(s_x, "x_scales", (torch.float32,), (M,), X.device)
    _call("zq_ln_quant_per_token", _ptr(X), _fdtype(X), M, K, pre, _ptr(gamma), _ptr(beta), eps,
          _ptr(Xq), _ptr(s_x), _stream(X))
    return Xq, s_x


def w8a8_gemm_dequant(Xq: torch.Tensor, x_scales: Optional[torch.Tensor], Wq: torch.Tensor,
                      w_scales: Optional[torch.Tensor], group_rows: int, bias=None,
                      act: int = ACT_NONE, out_dtype: torch.dtype = torch.float16,
                      path: int = PATH_AUTO, out: Optional[torch.Tensor] = None):
    """Y = dequant(Xq Wq^T) [+ bias] [GeLU], fp16.  out_dtype=torch.int32 returns the raw
    int32 accumulators (test mode)."""
    _need(Xq, "Xq", (torch.int8,))
    M, K = Xq.shape
    _need(Wq, "Wq", (torch.int8,), None, Xq.device)
    N = Wq.shape[0]
    if Wq.shape[1] != K:
        raise ValueError(f"Wq has K={Wq.shape[1]}, Xq has K={K}")
    if out_dtype == torch.float16:
        _need(x_scales, "x_scales", (torch.float32,), (M,), Xq.device)
        _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), Xq.device)
        ydt = F16
    elif out_dtype == torch.int32:
        ydt = I32
    else:
        raise TypeError("out_dtype must be torch.float16 or torch.int32")
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), Xq.device)
    Y = torch.empty((M, N), dtype=out_dtype, device=Xq.device) if out is None else out
    _need(Y, "out", (out_dtype,), (M, N), Xq.device)
    _call("zq_w8a8_gemm_dequant_ex", _ptr(Xq), _ptr(x_scales), _ptr(Wq), _ptr(w_scales),
          group_rows, _ptr(bias), act, M, N, K, _ptr(Y), ydt, path, _stream(Xq))
    return Y


def linear_workspace_bytes(M: int, K: int) -> int:
    return int(library().zq_linear_workspace_bytes(M, K))


def linear_w8a8(X: torch.Tensor, Wq: torch.Tensor, w_scales: torch.Tensor, group_rows: int,
                pre: int = PRE_LAYERNORM, gamma=None, beta=None, eps: float = 1e-5, bias=None,
                act: int = ACT_NONE, workspace: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None):
    """The fused layer: prologue (LN/GeLU + per-token quant) then GEMM + dequant -> fp16 [M, N]."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    _need(Wq, "Wq", (torch.int8,), None, X.device)
    N = Wq.shape[0]
    _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), X.device)
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), X.device)
    need = linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _need_ws(workspace, need, X.device)
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, N), X.device)
    _call("zq_linear_w8a8", _ptr(X), _fdtype(X), pre, _ptr(gamma), _ptr(beta), eps, _ptr(Wq),
          _ptr(w_scales), group_rows, _ptr(bias), act, M, N, K, _ptr(workspace),
          workspace.numel() * workspace.element_size(), _ptr(Y), _stream(X))
    return Y


NOALLOC_SCRATCH_BYTES = 32 << 20   # ZQ_NOALLOC_SCRATCH_BYTES in zq.h


def linear_w8a8_noalloc(X: torch.Tensor, Wq: torch.Tensor, w_scales: torch.Tensor,
                        group_rows: int, pre: int = PRE_LAYERNORM, gamma=None, beta=None,
                        eps: float = 1e-5, bias=None, act: int = ACT_NONE,
                        out: Optional[torch.Tensor] = None):
    """The fused layer with its codes and scales in the library's fixed per-GPU
    array (zq_linear_w8a8_noalloc): no workspace, nothing allocated by the call.
    Pass `out` to allocate nothing at all.  Calls that may overlap on one GPU race."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    _need(Wq, "Wq", (torch.int8,), None, X.device)
    N = Wq.shape[0]
    _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), X.device)
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), X.device)
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, N), X.device)
    with torch.cuda.device(X.device):
        _call("zq_linear_w8a8_noalloc", _ptr(X), _fdtype(X), pre, _ptr(gamma), _ptr(beta), eps,
              _ptr(Wq), _ptr(w_scales), group_rows, _ptr(bias), act, M, N, K, _ptr(Y), _stream(X))
    return Y


def linear_unfused_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(library().zq_linear_unfused_workspace_bytes(M, N, K))


def linear_w8a8_unfused(X: torch.Tensor, Wq: torch.Tensor, w_scales: torch.Tensor,
                        group_rows: int, pre: int = PRE_LAYERNORM, gamma=None, beta=None,
                        eps: float = 1e-5, bias=None, act: int = ACT_NONE,
                        workspace: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None):
    """The layer in the unfused order (op -> fp16 -> quantize -> int32 GEMM -> dequantize),
    for measuring the fusion gain.  The workspace holds the intermediates."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    _need(Wq, "Wq", (torch.int8,), None, X.device)
    N = Wq.shape[0]
    _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), X.device)
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), X.device)
    need = linear_unfused_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _need_ws(workspace, need, X.device)
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, N), X.device)
    _call("zq_linear_w8a8_unfused", _ptr(X), _fdtype(X), pre, _ptr(gamma), _ptr(beta), eps,
          _ptr(Wq), _ptr(w_scales), group_rows, _ptr(bias), act, M, N, K, _ptr(workspace),
          workspace.numel() * workspace.element_size(), _ptr(Y), _stream(X))
    return Y


def ffn_workspace_bytes(M: int, K: int, F: int) -> int:
    return int(library().zq_ffn_workspace_bytes(M, K, F))


def ffn_w8a8(X: torch.Tensor, W1q: torch.Tensor, w1_scales: torch.Tensor, group_rows1: int,
             W2q: torch.Tensor, w2_scales: torch.Tensor, group_rows2: int, gamma=None, beta=None,
             eps: float = 1e-5, bias1=None, bias2=None, workspace: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None):
    """FFN block: H = GeLU(linear(LN(X), W1) + b1), Y = linear(H, W2) + b2, chained; fp16 [M, K]."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    _need(W1q, "W1q", (torch.int8,), None, X.device)
    F = W1q.shape[0]
    if W1q.shape[1] != K:
        raise ValueError(f"W1q has K={W1q.shape[1]}, X has K={K}")
    _need(W2q, "W2q", (torch.int8,), (K, F), X.device)
    _need(w1_scales, "w1_scales", (torch.float32,), (F // group_rows1,), X.device)
    _need(w2_scales, "w2_scales", (torch.float32,), (K // group_rows2,), X.device)
    for name, t, n in (("gamma", gamma, K), ("beta", beta, K), ("bias1", bias1, F),
                       ("bias2", bias2, K)):
        if t is not None:
            _need(t, name, (torch.float32,), (n,), X.device)
    need = ffn_workspace_bytes(M, K, F)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _need_ws(workspace, need, X.device)
    Y = torch.empty((M, K), dtype=torch.float16, device=X.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, K), X.device)
    _call("zq_ffn_w8a8", _ptr(X), _fdtype(X), _ptr(gamma), _ptr(beta), eps, _ptr(W1q),
          _ptr(w1_scales), group_rows1, _ptr(bias1), _ptr(W2q), _ptr(w2_scales), group_rows2,
          _ptr(bias2), M, K, F, _ptr(workspace), workspace.numel() * workspace.element_size(),
          _ptr(Y), _stream(X))
    return Y


# ---- FP8 variant: OCP E4M3 codes (torch.uint8 tensors), power-of-two scales ----

def quantize_weights_grouped_fp8(W: torch.Tensor, group_rows: int,
                                 smooth: Optional[torch.Tensor] = None):
    """Offline group-wise FP8 codes of W [N, K] -> (uint8 codes [N, K], fp32 scales [N/G])."""
    _need(W, "W", (torch.float32, torch.float16))
    N, K = W.shape
    if smooth is not None:
        _need(smooth, "smooth", (torch.float32,), (K,), W.device)
    Wq = torch.empty((N, K), dtype=torch.uint8, device=W.device)
    s_w = torch.empty((max(N // group_rows, 1),), dtype=torch.float32, device=W.device)
    _call("zq_quantize_weights_grouped_fp8", _ptr(W), _fdtype(W), _ptr(smooth), N, K, group_rows,
          _ptr(Wq), _ptr(s_w), _stream(W))
    return Wq, s_w


def ln_quant_per_token_fp8(X: torch.Tensor, pre: int = PRE_LAYERNORM, gamma=None, beta=None,
                           eps: float = 1e-5):
    """Fused LN/GeLU + per-token FP8 codes -> (uint8 codes [M, K], fp32 power-of-two scales [M])."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    Xq = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    s_x = torch.empty((M,), dtype=torch.float32, device=X.device)
    _call("zq_ln_quant_per_token_fp8", _ptr(X), _fdtype(X), M, K, pre, _ptr(gamma), _ptr(beta),
          eps, _ptr(Xq), _ptr(s_x), _stream(X))
    return Xq, s_x


def fp8_gemm_dequant(Xq: torch.Tensor, x_scales: Optional[torch.Tensor], Wq: torch.Tensor,
                     w_scales: Optional[torch.Tensor], group_rows: int, bias=None,
                     act: int = ACT_NONE, out_dtype: torch.dtype = torch.float16):
    """FP8 GEMM + dequant -> fp16 [M, N]; out_dtype=torch.float32 returns the raw accumulators."""
    _need(Xq, "Xq", (torch.uint8,))
    M, K = Xq.shape
    _need(Wq, "Wq", (torch.uint8,), None, Xq.device)
    N = Wq.shape[0]
    if out_dtype == torch.float16:
        _need(x_scales, "x_scales", (torch.float32,), (M,), Xq.device)
        _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), Xq.device)
        ydt = F16
    elif out_dtype == torch.float32:
        ydt = F32
    else:
        raise TypeError("out_dtype must be torch.float16 or torch.float32")
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), Xq.device)
    Y = torch.empty((M, N), dtype=out_dtype, device=Xq.device)
    _call("zq_fp8_gemm_dequant", _ptr(Xq), _ptr(x_scales), _ptr(Wq), _ptr(w_scales), group_rows,
          _ptr(bias), act, M, N, K, _ptr(Y), ydt, _stream(Xq))
    return Y


def linear_w8a8_fp8(X: torch.Tensor, Wq: torch.Tensor, w_scales: torch.Tensor, group_rows: int,
                    pre: int = PRE_LAYERNORM, gamma=None, beta=None, eps: float = 1e-5, bias=None,
                    act: int = ACT_NONE, workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, N: Optional[int] = None,
                    packed: bool = False):
    """The FP8 layer -> fp16 [M, N].  With packed=True, Wq is zq_pack_weights' layout of the
    codes (M <= 32) and N must be given."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    if packed:
        if N is None:
            raise ValueError("packed weights need N")
        _need_packed(Wq.view(torch.int8), N, K, X.device)
    else:
        _need(Wq, "Wq", (torch.uint8,), None, X.device)
        N = Wq.shape[0]
    _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), X.device)
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), X.device)
    need = linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _need_ws(workspace, need, X.device)
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, N), X.device)
    _call("zq_linear_w8a8_fp8_packed" if packed else "zq_linear_w8a8_fp8", _ptr(X), _fdtype(X),
          pre, _ptr(gamma), _ptr(beta), eps, _ptr(Wq), _ptr(w_scales), group_rows, _ptr(bias),
          act, M, N, K, _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(Y),
          _stream(X))
    return Y


def packed_weights_bytes(N: int, K: int) -> int:
    return int(library().zq_packed_weights_bytes(N, K))


def pack_weights(Wq: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Offline re-layout of Wq int8 [N, K] into the packed layout zq.h defines
    (32-row x 512-byte blocks); returns a 1-D int8 tensor of
    packed_weights_bytes(N, K) bytes.  The packed calls take N explicitly."""
    _need(Wq, "Wq", (torch.int8, torch.uint8))
    N, K = Wq.shape
    nbytes = packed_weights_bytes(N, K)
    if nbytes == 0:
        raise ZQError("zq_pack_weights", 2)
    Wp = torch.empty((nbytes,), dtype=Wq.dtype, device=Wq.device) if out is None else out
    _need(Wp, "Wp", (torch.int8, torch.uint8), (nbytes,), Wq.device)
    _call("zq_pack_weights", _ptr(Wq), N, K, _ptr(Wp), _stream(Wq))
    return Wp


def _need_packed(Wp: torch.Tensor, N: int, K: int, device):
    _need(Wp, "Wp", (torch.int8,), None, device)
    if Wp.numel() != packed_weights_bytes(N, K):
        raise ValueError(f"Wp has {Wp.numel()} bytes, the packed layout of {N}x{K} has "
                         f"{packed_weights_bytes(N, K)}")


def w8a8_gemm_dequant_packed(Xq: torch.Tensor, x_scales: Optional[torch.Tensor], Wp: torch.Tensor,
                             w_scales: Optional[torch.Tensor], group_rows: int, N: int, bias=None,
                             act: int = ACT_NONE, out_dtype: torch.dtype = torch.float16,
                             out: Optional[torch.Tensor] = None):
    """As w8a8_gemm_dequant with packed weights (M <= 32)."""
    _need(Xq, "Xq", (torch.int8,))
    M, K = Xq.shape
    _need_packed(Wp, N, K, Xq.device)
    if out_dtype == torch.float16:
        _need(x_scales, "x_scales", (torch.float32,), (M,), Xq.device)
        _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), Xq.device)
        ydt = F16
    elif out_dtype == torch.int32:
        ydt = I32
    else:
        raise TypeError("out_dtype must be torch.float16 or torch.int32")
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), Xq.device)
    Y = torch.empty((M, N), dtype=out_dtype, device=Xq.device) if out is None else out
    _need(Y, "out", (out_dtype,), (M, N), Xq.device)
    _call("zq_w8a8_gemm_dequant_packed", _ptr(Xq), _ptr(x_scales), _ptr(Wp), _ptr(w_scales),
          group_rows, _ptr(bias), act, M, N, K, _ptr(Y), ydt, _stream(Xq))
    return Y


def linear_w8a8_packed(X: torch.Tensor, Wp: torch.Tensor, w_scales: torch.Tensor, group_rows: int,
                       N: int, pre: int = PRE_LAYERNORM, gamma=None, beta=None, eps: float = 1e-5,
                       bias=None, act: int = ACT_NONE, workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None):
    """As linear_w8a8 with packed weights (M <= 32)."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    _need_packed(Wp, N, K, X.device)
    _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), X.device)
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), X.device)
    need = linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _need_ws(workspace, need, X.device)
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, N), X.device)
    _call("zq_linear_w8a8_packed", _ptr(X), _fdtype(X), pre, _ptr(gamma), _ptr(beta), eps,
          _ptr(Wp), _ptr(w_scales), group_rows, _ptr(bias), act, M, N, K, _ptr(workspace),
          workspace.numel() * workspace.element_size(), _ptr(Y), _stream(X))
    return Y


def smoothquant_workspace_bytes(M: int, K: int) -> int:
    return int(library().zq_smoothquant_workspace_bytes(M, K))


def smoothquant_factors(X: torch.Tensor, W: torch.Tensor, eps: float = 1e-5, gamma=None, beta=None):
    """Offline SmoothQuant calibration on X [M, K] and W [N, K].
    Returns (smooth [K], gamma_out [K], beta_out [K]), all fp32."""
    _need(X, "X", (torch.float32, torch.float16))
    _need(W, "W", (torch.float32, torch.float16), None, X.device)
    M, K = X.shape
    N = W.shape[0]
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    s = torch.empty((K,), dtype=torch.float32, device=X.device)
    g = torch.empty_like(s)
    b = torch.empty_like(s)
    need = smoothquant_workspace_bytes(M, K)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _call("zq_smoothquant_factors", _ptr(X), _fdtype(X), M, K, eps, _ptr(W), _fdtype(W), N,
          _ptr(gamma), _ptr(beta), _ptr(s), _ptr(g), _ptr(b), _ptr(ws), need, _stream(X))
    return s, g, b


# ---- Mixed-precision decomposition (outlier columns in fp16) ----

def pack_outlier_weights(W: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Offline: W [N, K] (fp32/fp16) -> fp16 [K, N] (W transposed, nearest-even)."""
    _need(W, "W", (torch.float32, torch.float16))
    N, K = W.shape
    Wt = torch.empty((K, N), dtype=torch.float16, device=W.device) if out is None else out
    _need(Wt, "out", (torch.float16,), (K, N), W.device)
    _call("zq_pack_outlier_weights", _ptr(W), _fdtype(W), N, K, _ptr(Wt), _stream(W))
    return Wt


def outlier_columns(X: torch.Tensor, alpha: float = 6.0, pre: int = PRE_LAYERNORM, gamma=None,
                    beta=None, eps: float = 1e-5,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Outlier set of the batch -> (slot int32 [K], cols int32 [K + 1]):
    cols[0] = |O|, cols[1:1+|O|] ascending; slot[j] = position of j in O or -1."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if out is None:
        slot = torch.empty((K,), dtype=torch.int32, device=X.device)
        cols = torch.empty((K + 1,), dtype=torch.int32, device=X.device)
    else:
        slot, cols = out
    _need(slot, "slot", (torch.int32,), (K,), X.device)
    _need(cols, "cols", (torch.int32,), (K + 1,), X.device)
    _call("zq_outlier_columns", _ptr(X), _fdtype(X), M, K, pre, _ptr(gamma), _ptr(beta), eps,
          alpha, _ptr(slot), _ptr(cols), _stream(X))
    return slot, cols


def ln_quant_decomp(X: torch.Tensor, slot: torch.Tensor, pre: int = PRE_LAYERNORM, gamma=None,
                    beta=None, eps: float = 1e-5,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Prologue of the INT8 part over the non-outlier columns ->
    (Xq int8 [M, K], s_x fp32 [M], XO fp16 [M, K]; XO[m, p] = y of the p-th outlier column)."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    _need(slot, "slot", (torch.int32,), (K,), X.device)
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if out is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
        s_x = torch.empty((M,), dtype=torch.float32, device=X.device)
        XO = torch.empty((M, K), dtype=torch.float16, device=X.device)
    else:
        Xq, s_x, XO = out
    _need(Xq, "Xq", (torch.int8,), (M, K), X.device)
    _need(s_x, "s_x", (torch.float32,), (M,), X.device)
    _need(XO, "XO", (torch.float16,), (M, K), X.device)
    _call("zq_ln_quant_decomp", _ptr(X), _fdtype(X), M, K, pre, _ptr(gamma), _ptr(beta), eps,
          _ptr(slot), _ptr(Xq), _ptr(s_x), _ptr(XO), _stream(X))
    return Xq, s_x, XO


def w8a8_gemm_decomp(Xq: torch.Tensor, x_scales: torch.Tensor, Wq: torch.Tensor,
                     w_scales: torch.Tensor, group_rows: int, cols: torch.Tensor, XO: torch.Tensor,
                     W16t: torch.Tensor, bias=None, act: int = ACT_NONE,
                     out: Optional[torch.Tensor] = None):
    """INT8 GEMM + dequant + FP16 outlier product (+bias, GeLU) -> fp16 [M, N]."""
    _need(Xq, "Xq", (torch.int8,))
    M, K = Xq.shape
    _need(Wq, "Wq", (torch.int8,), None, Xq.device)
    N = Wq.shape[0]
    _need(x_scales, "x_scales", (torch.float32,), (M,), Xq.device)
    _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), Xq.device)
    _need(cols, "cols", (torch.int32,), (K + 1,), Xq.device)
    _need(XO, "XO", (torch.float16,), (M, K), Xq.device)
    _need(W16t, "W16t", (torch.float16,), (K, N), Xq.device)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), Xq.device)
    Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, N), Xq.device)
    _call("zq_w8a8_gemm_decomp", _ptr(Xq), _ptr(x_scales), _ptr(Wq), _ptr(w_scales), group_rows,
          _ptr(cols), _ptr(XO), _ptr(W16t), _ptr(bias), act, M, N, K, _ptr(Y), _stream(Xq))
    return Y


def linear_decomp_workspace_bytes(M: int, K: int) -> int:
    return int(library().zq_linear_decomp_workspace_bytes(M, K))


def linear_w8a8_decomp(X: torch.Tensor, Wq: torch.Tensor, w_scales: torch.Tensor, group_rows: int,
                       W16t: torch.Tensor, alpha: float = 6.0, pre: int = PRE_LAYERNORM,
                       gamma=None, beta=None, eps: float = 1e-5, bias=None, act: int = ACT_NONE,
                       workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None):
    """The decomposed layer (outlier columns in fp16, the rest W8A8) -> fp16 [M, N]."""
    _need(X, "X", (torch.float32, torch.float16))
    M, K = X.shape
    _need(Wq, "Wq", (torch.int8,), None, X.device)
    N = Wq.shape[0]
    _need(w_scales, "w_scales", (torch.float32,), (N // group_rows,), X.device)
    _need(W16t, "W16t", (torch.float16,), (K, N), X.device)
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _need(t, name, (torch.float32,), (K,), X.device)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), (N,), X.device)
    need = linear_decomp_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _need_ws(workspace, need, X.device)
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device) if out is None else out
    _need(Y, "out", (torch.float16,), (M, N), X.device)
    _call("zq_linear_w8a8_decomp", _ptr(X), _fdtype(X), pre, _ptr(gamma), _ptr(beta), eps, alpha,
          _ptr(Wq), _ptr(w_scales), group_rows, _ptr(W16t), _ptr(bias), act, M, N, K,
          _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(Y), _stream(X))
    return Y
