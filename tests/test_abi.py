"""The C ABI: the library loads, exports every entry point zq.h declares, and
rejects bad arguments on the host before touching the GPU.  Runs on the CPU
(fake, never-dereferenced pointers; validation happens before any HIP call)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

import post_w8a8_quantized_amd as zq
from post_w8a8_quantized_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 1 << 20          # a fake 16-byte-aligned address; never dereferenced
UNALIGNED = A + 4

OK, NULL, SHAPE, ALIGN, DTYPE, WS, HIP = 0, 1, 2, 3, 4, 5, 6


@pytest.fixture(scope="module")
def L():
    return zq.library()


def test_library_exports_every_declared_symbol(L):
    names = zq.exported_symbols()
    assert len(names) == 29
    out = subprocess.run(["nm", "-D", "--defined-only", zq.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)
    # Nothing beyond the declared API is exported.
    assert {n for n in exported if n.startswith("zq")} == set(names)


def test_single_hip_runtime_mapped(L):
    assert len(B._hip_runtimes_mapped()) <= 1


def test_status_strings(L):
    for s in range(8):
        assert L.zq_status_str(s).decode().startswith(B._STATUS[s])
    assert L.zq_status_str(99) == b"unknown zq_status"


def test_workspace_sizes(L):
    assert L.zq_linear_workspace_bytes(4096, 768) == 4096 * 768 + 4 * 4096
    assert L.zq_linear_workspace_bytes(3, 16) == 256 + 256
    assert L.zq_linear_workspace_bytes(0, 16) == 0
    assert L.zq_linear_workspace_bytes(4, 17) == 0
    assert L.zq_smoothquant_workspace_bytes(4096, 5120) == 8 * 4096 + 8 * 5120
    assert L.zq_smoothquant_workspace_bytes(1, 16) == 256


def gemm(L, Xq=A, sx=A, Wq=A, sw=A, G=128, bias=None, act=0, M=16, N=256, K=256, Y=A, ydt=1,
         path=0):
    return L.zq_w8a8_gemm_dequant_ex(Xq, sx, Wq, sw, G, bias, act, M, N, K, Y, ydt, path, None)


@pytest.mark.parametrize("kw,want", [
    (dict(Xq=None), NULL), (dict(Wq=None), NULL), (dict(Y=None), NULL),
    (dict(sx=None), NULL), (dict(sw=None), NULL),
    (dict(M=0), SHAPE), (dict(N=0), SHAPE), (dict(K=0), SHAPE), (dict(K=24), SHAPE),
    (dict(K=131072 + 16), SHAPE), (dict(G=0), SHAPE), (dict(G=96), SHAPE),
    (dict(N=250, G=2), SHAPE), (dict(M=33, path=2), SHAPE),
    (dict(M=1 << 31, K=16), SHAPE), (dict(N=1 << 31, K=16, G=1), SHAPE),
    (dict(M=1 << 21, N=1 << 20, K=16, G=1), SHAPE),    # Y would exceed 2^40 elements
    (dict(M=1 << 24, K=1 << 17), SHAPE),                # Xq would exceed 2^40 elements
    (dict(Xq=UNALIGNED), ALIGN), (dict(Wq=UNALIGNED), ALIGN), (dict(Y=UNALIGNED), ALIGN),
    (dict(ydt=0), DTYPE), (dict(ydt=2), DTYPE), (dict(act=2), DTYPE), (dict(path=3), DTYPE),
])
def test_gemm_validation(L, kw, want):
    assert gemm(L, **kw) == want


def test_gemm_i32_mode_does_not_need_scales(L):
    # Valid in test mode without scales: passes validation and reaches the launch,
    # which fails only where there is no GPU.
    st = gemm(L, sx=None, sw=None, ydt=3)
    assert st in (OK, HIP) and (st == HIP) == (not os.path.exists("/dev/kfd"))


def prologue(L, X=A, dt=1, M=8, K=256, pre=1, g=None, b=None, Xq=A, sx=A):
    return L.zq_ln_quant_per_token(X, dt, M, K, pre, g, b, 1e-5, Xq, sx, None)


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(Xq=None), NULL), (dict(sx=None), NULL),
    (dict(dt=2), DTYPE), (dict(dt=3), DTYPE), (dict(pre=3), DTYPE),
    (dict(M=0), SHAPE), (dict(K=8), SHAPE), (dict(K=0), SHAPE), (dict(K=262144), SHAPE),
    (dict(X=UNALIGNED), ALIGN), (dict(Xq=UNALIGNED), ALIGN), (dict(g=UNALIGNED), ALIGN),
])
def test_prologue_validation(L, kw, want):
    assert prologue(L, **kw) == want


def test_prologue_ignores_gamma_alignment_without_layernorm(L):
    st = prologue(L, pre=2, g=UNALIGNED)
    assert st in (OK, HIP)


def linear(L, X=A, dt=1, pre=1, Wq=A, sw=A, G=128, M=16, N=256, K=256, ws=A, wsb=1 << 30, Y=A,
           act=0):
    return L.zq_linear_w8a8(X, dt, pre, None, None, 1e-5, Wq, sw, G, None, act, M, N, K, ws, wsb, Y,
                            None)


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(Wq=None), NULL), (dict(sw=None), NULL), (dict(Y=None), NULL),
    (dict(ws=None), WS), (dict(wsb=16 * 256), WS), (dict(ws=A + 16), ALIGN),
    (dict(K=40), SHAPE), (dict(G=100), SHAPE), (dict(M=0), SHAPE), (dict(dt=3), DTYPE),
    (dict(act=5), DTYPE), (dict(X=UNALIGNED), ALIGN),
])
def test_linear_validation(L, kw, want):
    assert linear(L, **kw) == want


def test_linear_workspace_exact_size_accepted(L):
    need = L.zq_linear_workspace_bytes(16, 256)
    assert linear(L, wsb=need) in (OK, HIP)
    assert linear(L, wsb=need - 1) == WS


@pytest.mark.parametrize("kw,want", [
    (dict(W=None), NULL), (dict(Wq=None), NULL), (dict(s=None), NULL), (dict(dt=2), DTYPE),
    (dict(N=0), SHAPE), (dict(G=3), SHAPE), (dict(K=20), SHAPE), (dict(W=UNALIGNED), ALIGN),
])
def test_weight_quant_validation(L, kw, want):
    a = dict(W=A, dt=0, smooth=None, N=256, K=256, G=64, Wq=A, s=A)
    a.update(kw)
    assert L.zq_quantize_weights_grouped(a["W"], a["dt"], a["smooth"], a["N"], a["K"], a["G"],
                                         a["Wq"], a["s"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(W=None), NULL), (dict(s=None), NULL), (dict(xdt=2), DTYPE),
    (dict(wdt=3), DTYPE), (dict(K=12), SHAPE), (dict(N=0), SHAPE), (dict(ws=None), WS),
    (dict(wsb=10), WS), (dict(X=UNALIGNED), ALIGN), (dict(ws=A + 64), ALIGN),
])
def test_smooth_validation(L, kw, want):
    a = dict(X=A, xdt=1, M=64, K=128, W=A, wdt=0, N=32, s=A, ws=A, wsb=1 << 20)
    a.update(kw)
    assert L.zq_smoothquant_factors(a["X"], a["xdt"], a["M"], a["K"], 1e-5, a["W"], a["wdt"],
                                    a["N"], None, None, a["s"], A, A, a["ws"], a["wsb"],
                                    None) == want


def test_packed_weight_sizes(L):
    # ceil(N / 32) * 32 rows by ceil(K / 512) * 512 bytes.
    assert L.zq_packed_weights_bytes(8192, 28672) == 8192 * 28672
    assert L.zq_packed_weights_bytes(100, 208) == 128 * 512
    assert L.zq_packed_weights_bytes(32, 528) == 32 * 1024
    assert L.zq_packed_weights_bytes(0, 512) == 0
    assert L.zq_packed_weights_bytes(32, 24) == 0
    assert L.zq_packed_weights_bytes(32, 131072 + 16) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(Wq=None), NULL), (dict(Wp=None), NULL), (dict(N=0), SHAPE), (dict(K=40), SHAPE),
    (dict(Wq=UNALIGNED), ALIGN), (dict(Wp=UNALIGNED), ALIGN),
])
def test_pack_validation(L, kw, want):
    a = dict(Wq=A, N=64, K=512, Wp=A)
    a.update(kw)
    assert L.zq_pack_weights(a["Wq"], a["N"], a["K"], a["Wp"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(Xq=None), NULL), (dict(Wp=None), NULL), (dict(M=33), SHAPE), (dict(K=24), SHAPE),
    (dict(N=250, G=2), SHAPE), (dict(Wp=UNALIGNED), ALIGN), (dict(ydt=0), DTYPE),
])
def test_gemm_packed_validation(L, kw, want):
    a = dict(Xq=A, sx=A, Wp=A, sw=A, G=128, M=16, N=256, K=256, Y=A, ydt=1)
    a.update(kw)
    assert L.zq_w8a8_gemm_dequant_packed(a["Xq"], a["sx"], a["Wp"], a["sw"], a["G"], None, 0,
                                         a["M"], a["N"], a["K"], a["Y"], a["ydt"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(Wp=None), NULL), (dict(M=33), SHAPE), (dict(ws=None), WS), (dict(wsb=16), WS),
])
def test_linear_packed_validation(L, kw, want):
    a = dict(Wp=A, M=16, ws=A, wsb=1 << 30)
    a.update(kw)
    assert L.zq_linear_w8a8_packed(A, 1, 1, None, None, 1e-5, a["Wp"], A, 128, None, 0, a["M"],
                                   256, 256, a["ws"], a["wsb"], A, None) == want


def test_unfused_workspace_sizes(L):
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert L.zq_linear_unfused_workspace_bytes(4096, 3072, 768) == \
        r(2 * 4096 * 768) + r(4096 * 768) + r(4 * 4096) + r(4 * 4096 * 3072)
    assert L.zq_linear_unfused_workspace_bytes(3, 4, 16) == 256 * 4
    assert L.zq_linear_unfused_workspace_bytes(3, 0, 16) == 0
    assert L.zq_linear_unfused_workspace_bytes(3, 4, 20) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(Wq=None), NULL), (dict(ws=None), WS), (dict(wsb=4096), WS),
    (dict(ws=A + 16), ALIGN), (dict(K=40), SHAPE), (dict(act=4), DTYPE), (dict(X=UNALIGNED), ALIGN),
])
def test_unfused_validation(L, kw, want):
    a = dict(X=A, Wq=A, M=16, N=256, K=256, ws=A, wsb=1 << 30, act=0)
    a.update(kw)
    assert L.zq_linear_w8a8_unfused(a["X"], 1, 1, None, None, 1e-5, a["Wq"], A, 128, None,
                                    a["act"], a["M"], a["N"], a["K"], a["ws"], a["wsb"], A,
                                    None) == want


def test_ffn_workspace_sizes(L):
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    M, K, F = 4096, 768, 3072
    assert L.zq_ffn_workspace_bytes(M, K, F) == \
        r(M * K) + r(4 * M) + r(2 * M * F) + r(4 * M * (F // 16 + 2)) + r(M * F) + r(4 * M)
    assert L.zq_ffn_workspace_bytes(1, 16, 16) == 6 * 256
    assert L.zq_ffn_workspace_bytes(1, 16, 24) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(W1=None), NULL), (dict(W2=None), NULL), (dict(ws=None), WS),
    (dict(wsb=4096), WS), (dict(F=40), SHAPE), (dict(G2=100), SHAPE), (dict(G1=5), SHAPE),
    (dict(X=UNALIGNED), ALIGN), (dict(W2=UNALIGNED), ALIGN),
])
def test_ffn_validation(L, kw, want):
    a = dict(X=A, W1=A, W2=A, G1=128, G2=128, M=16, K=256, F=1024, ws=A, wsb=1 << 30)
    a.update(kw)
    assert L.zq_ffn_w8a8(a["X"], 1, None, None, 1e-5, a["W1"], A, a["G1"], None, a["W2"], A,
                         a["G2"], None, a["M"], a["K"], a["F"], a["ws"], a["wsb"], A,
                         None) == want


def test_decomp_workspace_sizes(L):
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    M, K = 4096, 5120
    assert L.zq_linear_decomp_workspace_bytes(M, K) == \
        r(4 * K) + r(4 * (K + 1)) + r(M * K) + r(4 * M) + r(2 * M * K)
    assert L.zq_linear_decomp_workspace_bytes(1, 16) == 5 * 256
    assert L.zq_linear_decomp_workspace_bytes(0, 16) == 0
    assert L.zq_linear_decomp_workspace_bytes(4, 24) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(Wq=None), NULL), (dict(sw=None), NULL), (dict(Wt=None), NULL),
    (dict(Y=None), NULL), (dict(ws=None), WS), (dict(wsb=4096), WS), (dict(ws=A + 16), ALIGN),
    (dict(K=40), SHAPE), (dict(G=100), SHAPE), (dict(M=0), SHAPE), (dict(dt=3), DTYPE),
    (dict(pre=3), DTYPE), (dict(act=5), DTYPE), (dict(X=UNALIGNED), ALIGN),
    (dict(Wt=UNALIGNED), ALIGN),
])
def test_linear_decomp_validation(L, kw, want):
    a = dict(X=A, dt=1, pre=1, Wq=A, sw=A, G=128, Wt=A, M=16, N=256, K=256, ws=A, wsb=1 << 30,
             Y=A, act=0)
    a.update(kw)
    assert L.zq_linear_w8a8_decomp(a["X"], a["dt"], a["pre"], None, None, 1e-5, 6.0, a["Wq"],
                                   a["sw"], a["G"], a["Wt"], None, a["act"], a["M"], a["N"],
                                   a["K"], a["ws"], a["wsb"], a["Y"], None) == want


def test_linear_decomp_workspace_exact_size_accepted(L):
    need = L.zq_linear_decomp_workspace_bytes(16, 256)
    call = lambda wsb: L.zq_linear_w8a8_decomp(A, 1, 1, None, None, 1e-5, 6.0, A, A, 128, A,  # noqa: E731
                                               None, 0, 16, 256, 256, A, wsb, A, None)
    assert call(need) in (OK, HIP)
    assert call(need - 1) == WS


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(slot=None), NULL), (dict(cols=None), NULL),
    (dict(K=24), SHAPE), (dict(M=0), SHAPE), (dict(dt=2), DTYPE), (dict(pre=7), DTYPE),
    (dict(X=UNALIGNED), ALIGN), (dict(slot=UNALIGNED), ALIGN),
])
def test_outlier_columns_validation(L, kw, want):
    a = dict(X=A, dt=1, pre=1, M=16, K=256, slot=A, cols=A)
    a.update(kw)
    assert L.zq_outlier_columns(a["X"], a["dt"], a["M"], a["K"], a["pre"], None, None, 1e-5, 6.0,
                                a["slot"], a["cols"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(slot=None), NULL), (dict(Xq=None), NULL), (dict(sx=None), NULL),
    (dict(XO=None), NULL), (dict(K=24), SHAPE), (dict(XO=UNALIGNED), ALIGN),
    (dict(slot=UNALIGNED), ALIGN), (dict(Xq=UNALIGNED), ALIGN),
])
def test_ln_quant_decomp_validation(L, kw, want):
    a = dict(X=A, M=16, K=256, slot=A, Xq=A, sx=A, XO=A)
    a.update(kw)
    assert L.zq_ln_quant_decomp(a["X"], 1, a["M"], a["K"], 1, None, None, 1e-5, a["slot"], a["Xq"],
                                a["sx"], a["XO"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(Xq=None), NULL), (dict(sx=None), NULL), (dict(cols=None), NULL), (dict(XO=None), NULL),
    (dict(Wt=None), NULL), (dict(Y=None), NULL), (dict(N=250, G=2), SHAPE), (dict(K=40), SHAPE),
    (dict(act=2), DTYPE), (dict(XO=UNALIGNED), ALIGN), (dict(Wt=UNALIGNED), ALIGN),
])
def test_gemm_decomp_validation(L, kw, want):
    a = dict(Xq=A, sx=A, G=128, cols=A, XO=A, Wt=A, act=0, M=16, N=256, K=256, Y=A)
    a.update(kw)
    assert L.zq_w8a8_gemm_decomp(a["Xq"], a["sx"], A, A, a["G"], a["cols"], a["XO"], a["Wt"], None,
                                 a["act"], a["M"], a["N"], a["K"], a["Y"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(W=None), NULL), (dict(Wt=None), NULL), (dict(dt=2), DTYPE), (dict(N=0), SHAPE),
    (dict(K=20), SHAPE), (dict(W=UNALIGNED), ALIGN), (dict(Wt=UNALIGNED), ALIGN),
])
def test_pack_outlier_weights_validation(L, kw, want):
    a = dict(W=A, dt=0, N=256, K=256, Wt=A)
    a.update(kw)
    assert L.zq_pack_outlier_weights(a["W"], a["dt"], a["N"], a["K"], a["Wt"], None) == want


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="checks the no-GPU error path")
def test_valid_call_without_gpu_reports_hip_error(L):
    assert gemm(L) == HIP
    assert prologue(L) == HIP


def test_binding_rejects_cpu_tensors():
    import torch
    X = torch.zeros((4, 16), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        zq.ln_quant_per_token(X)


def noalloc(L, X=A, dt=1, pre=1, Wq=A, sw=A, G=128, M=16, N=256, K=256, Y=A, act=0):
    return L.zq_linear_w8a8_noalloc(X, dt, pre, None, None, 1e-5, Wq, sw, G, None, act, M, N, K, Y,
                                    None)


@pytest.mark.parametrize("kw,want", [
    (dict(X=None), NULL), (dict(Wq=None), NULL), (dict(sw=None), NULL), (dict(Y=None), NULL),
    (dict(K=24), SHAPE), (dict(M=0), SHAPE),
    (dict(M=8200, K=4096), WS),            # codes + scales beyond the 32 MiB array
])
def test_noalloc_validation(L, kw, want):
    assert noalloc(L, **kw) == want


def test_noalloc_limit(L):
    # the largest token count whose codes and scales fit at K = 4096
    lim = 32 << 20
    assert L.zq_linear_workspace_bytes(8176, 4096) <= lim < L.zq_linear_workspace_bytes(8200, 4096)


def test_binding_checks_workspace_tensor():
    """The C ABI sees only a pointer and a byte count, so the binding rejects a
    workspace on the host, on another device, non-contiguous or too small."""
    import torch
    gpu = torch.device("cuda:0")
    with pytest.raises(ValueError, match="workspace is on cpu"):
        B._need_ws(torch.zeros(1024, dtype=torch.uint8), 512, gpu)
    with pytest.raises(TypeError):
        B._need_ws(None, 512, gpu)
    with pytest.raises(ValueError, match="GPU"):
        B._need(torch.zeros((4, 4), dtype=torch.float16), "out", (torch.float16,), (4, 4))


def test_gemm_rejects_n_not_multiple_of_4(L):
    """N % 4 == 0 (outputs are written four columns at a time), for every call
    that runs the GEMM, in test mode too."""
    assert gemm(L, N=250, G=2) == SHAPE
    assert gemm(L, N=250, G=2, ydt=3, sx=None, sw=None) == SHAPE
    assert gemm(L, N=6, G=1) == SHAPE
    assert linear(L, N=250, G=2) == SHAPE


def test_missing_library_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(zq.ZQError, match="not built"):
        B.library()
