"""The chained FFN block: bit-identical to two zq_linear_w8a8 calls (FFN-up with
LayerNorm and the GeLU epilogue, then FFN-down without a pre-op on H), the
scales of H (from the partial row maxima the FFN-up epilogue writes) equal to
fl32(max |H| / 127) exactly, and the block against the oracle's chain."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from tests._match import assert_y, say
from zq_workloads import random_affine

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def zq():
    import post_w8a8_quantized_amd as m
    assert torch.cuda.is_available(), "a GPU device node exists but torch sees no GPU"
    m.library()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def r256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("M,K,F,dt", [
    (16, 256, 1024, np.float32),    # weight-streaming kernels
    (5, 768, 3072, np.float16),
    (200, 768, 3072, np.float16),   # tiled kernels, ragged M
    (300, 512, 1040, np.float16),   # ragged F tile
    (40, 256, 4112, np.float16),    # H rows longer than the quantizer holds in registers
])
def test_ffn_block(zq, M, K, F, dt):
    say("ffn", M, K, F, dt.__name__)
    rng = np.random.default_rng(M + K + F)
    X = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(dt)
    g, b = random_affine(rng, K)
    W1 = (0.02 * rng.standard_normal((F, K))).astype(np.float32)
    W2 = (0.02 * rng.standard_normal((K, F))).astype(np.float32)
    b1 = (0.01 * rng.standard_normal(F)).astype(np.float32)
    b2 = (0.01 * rng.standard_normal(K)).astype(np.float32)
    G1, G2 = 16, 16
    W1q, s1 = zq.quantize_weights_grouped(dev(W1), G1)
    W2q, s2 = zq.quantize_weights_grouped(dev(W2), G2)
    Xd, gd, bd, b1d, b2d = dev(X), dev(g), dev(b), dev(b1), dev(b2)
    ws = torch.zeros(zq.ffn_workspace_bytes(M, K, F), dtype=torch.uint8, device="cuda")
    Y = host(zq.ffn_w8a8(Xd, W1q, s1, G1, W2q, s2, G2, gd, bd, 1e-5, b1d, b2d, workspace=ws))

    # two separate layer calls
    H2 = zq.linear_w8a8(Xd, W1q, s1, G1, zq.PRE_LAYERNORM, gd, bd, 1e-5, b1d, zq.ACT_GELU)
    Y2 = host(zq.linear_w8a8(H2, W2q, s2, G2, zq.PRE_NONE, None, None, 1e-5, b2d, zq.ACT_NONE))
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))

    # H in the workspace, and H's per-token scales, which come from the partial
    # row maxima the FFN-up epilogue wrote: exactly fl32(max |H[m, :]| / 127)
    w = host(ws)
    off = r256(M * K) + r256(4 * M)
    H = w[off:off + 2 * M * F].view(np.float16).reshape(M, F)
    assert np.array_equal(H.view(np.uint16), host(H2).view(np.uint16))
    off += r256(2 * M * F) + r256(4 * M * (F // 16 + 2)) + r256(M * F)
    sx2 = w[off:off + 4 * M].view(np.float32)
    amax = np.max(np.abs(H.astype(np.float32)), axis=1)
    assert np.array_equal(sx2, (amax / np.float32(127.0)).astype(np.float32))

    # against the oracle's chain (its own H, codes and scales)
    W1q_h, s1_h, W2q_h, s2_h = host(W1q), host(s1), host(W2q), host(s2)
    H_ref = ref.linear(X, ref.PRE_LAYERNORM, g, b, 1e-5, W1q_h, s1_h, G1, b1, ref.ACT_GELU)[0]
    Y_ref = ref.linear(H_ref, ref.PRE_NONE, None, None, 1e-5, W2q_h, s2_h, G2, b2,
                       ref.ACT_NONE)[0]
    assert_y(Y, Y_ref)
