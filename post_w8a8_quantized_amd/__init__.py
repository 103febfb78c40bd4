"""post_w8a8_quantized_amd -- ZeroQuant-style W8A8 linear layers on MI355X (gfx950).

A thin Python binding over the C ABI of libzq.so (include/zq.h).  Each
function has the name of the C entry point it calls, takes torch tensors that
live on the GPU, checks their device, dtype, shape and contiguity, and passes
raw device pointers plus torch's current HIP stream.  All arithmetic runs in
the library's HIP kernels; there is no fallback.  If the library is missing
or cannot be loaded, every call raises.

    import torch, post_w8a8_quantized_amd as zq
    Wq, s_w = zq.quantize_weights_grouped(W, group_rows=128)       # offline
    Y = zq.linear_w8a8(X, Wq, s_w, 128, pre=zq.PRE_LAYERNORM, bias=b)

Offline weight preparation and the SmoothQuant fold are also exposed
(`smoothquant_factors`, `quantize_weights_grouped(..., smooth=s)`), and for
decode shapes (M <= 32) the weights can be re-laid out once with
`pack_weights` and used by `linear_w8a8_packed` / `w8a8_gemm_dequant_packed`.
The mixed-precision decomposition (outlier columns in fp16, LLM.int8()) is
`linear_w8a8_decomp`, with its fp16 weights from `pack_outlier_weights`.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    ACT_GELU,
    ACT_NONE,
    PATH_AUTO,
    PATH_SKINNY,
    PATH_TILED,
    PRE_GELU,
    PRE_LAYERNORM,
    PRE_NONE,
    ZQError,
    exported_symbols,
    ffn_w8a8,
    ffn_workspace_bytes,
    fp8_gemm_dequant,
    library,
    library_path,
    linear_decomp_workspace_bytes,
    linear_w8a8_decomp,
    ln_quant_decomp,
    outlier_columns,
    pack_outlier_weights,
    w8a8_gemm_decomp,
    linear_w8a8,
    linear_w8a8_noalloc,
    NOALLOC_SCRATCH_BYTES,
    linear_unfused_workspace_bytes,
    linear_w8a8_fp8,
    linear_w8a8_packed,
    linear_w8a8_unfused,
    linear_workspace_bytes,
    ln_quant_per_token,
    ln_quant_per_token_fp8,
    pack_weights,
    packed_weights_bytes,
    quantize_weights_grouped,
    quantize_weights_grouped_fp8,
    smoothquant_factors,
    smoothquant_workspace_bytes,
    w8a8_gemm_dequant,
    w8a8_gemm_dequant_packed,
)

__all__ = [
    "ACT_GELU", "ACT_NONE", "PATH_AUTO", "PATH_SKINNY", "PATH_TILED", "PRE_GELU",
    "PRE_LAYERNORM", "PRE_NONE", "ZQError", "exported_symbols", "ffn_w8a8", "ffn_workspace_bytes",
    "fp8_gemm_dequant", "linear_w8a8_fp8", "ln_quant_per_token_fp8", "quantize_weights_grouped_fp8",
    "library", "library_path",
    "linear_decomp_workspace_bytes", "linear_w8a8_decomp", "ln_quant_decomp", "outlier_columns",
    "pack_outlier_weights", "w8a8_gemm_decomp",
    "linear_unfused_workspace_bytes", "linear_w8a8", "linear_w8a8_noalloc",
    "NOALLOC_SCRATCH_BYTES", "linear_w8a8_packed", "linear_w8a8_unfused",
    "linear_workspace_bytes", "ln_quant_per_token",
    "pack_weights", "packed_weights_bytes", "quantize_weights_grouped", "smoothquant_factors",
    "smoothquant_workspace_bytes", "w8a8_gemm_dequant", "w8a8_gemm_dequant_packed",
]
