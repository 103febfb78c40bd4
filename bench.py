"""Benchmark of the W8A8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the per-token hot path over one batch: the fused
LayerNorm/GeLU + per-token quantization kernel, then the int8 MFMA GEMM with
the fused dequant (+bias, +GeLU) epilogue, through zq_linear_w8a8.  Weights
are quantized offline (by the library) before timing, as the method
prescribes.  Inputs are seeded synthetic data resident in HBM; several
independent input/weight/output sets are rotated so that the 256 MB
Infinity Cache cannot serve a step from the previous one.

The steps are captured in a HIP graph (on torch's stream, which is the
stream the library launches on) so that host-side call overhead does not
leave the GPU idle between the ~10 us layers; the timed region is one replay
of a graph of exactly K steps, bracketed by device synchronisations.

Printed: ONE JSON line with the throughput (TOPS for prefill workloads, GB/s
for the decode workload), the dominant kernel's roofline figures measured
with HIP events, and the CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 fused linear TOPS (% int8 MFMA peak) prefill; GB/s (% HBM) decode"
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
PRE_NAMES = {0: "none", 1: "layernorm", 2: "gelu"}
ACT_NAMES = {0: "none", 1: "gelu"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="bert_ffn_up")
    ap.add_argument("--rotate-mb", type=float, default=600.0,
                    help="total bytes of the rotated input sets (beyond the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the unfused-order comparison (prefill workloads)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 (E4M3, power-of-two scales) variant timing")
    ap.add_argument("--no-decomp", action="store_true",
                    help="skip the outlier-workload leg (SmoothQuant fold vs the LLM.int8() "
                         "mixed-precision decomposition)")
    ap.add_argument("--no-ffn", action="store_true",
                    help="skip the chained FFN block timing (bert_ffn_up)")
    ap.add_argument("--no-copy-reference", action="store_true",
                    help="skip the 1 GiB device-copy bandwidth reference")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat full oracle passes until this much wall time has passed")
    ap.add_argument("--calib-copy-mb", type=float, default=0.0,
                    help="only run a plain device copy of this size (counter calibration)")
    return ap.parse_args()


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "post_w8a8_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def graph_of(torch, fn, n):
    """Capture n calls fn(i) into one graph (after two eager warm calls on a side stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
        fn(1 % max(n, 1))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g):
    """Milliseconds for one replay, bracketed by device synchronisations."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return e0.elapsed_time(e1), wall


def calib_copy(torch, mb):
    n = int(mb * 1024 * 1024)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 5}), flush=True)


def outlier_leg(torch, zq, w, make_inputs, args, dev):
    """Times the outlier workload with the SmoothQuant fold (fused layer) and with
    the mixed-precision decomposition, plus the decomposition's stages."""
    inp = make_inputs(w)
    M, N, K = w.M, w.N, w.K
    Xd = torch.from_numpy(inp.X).to(dev)
    Wd = torch.from_numpy(inp.W).to(dev)
    gamma = torch.from_numpy(inp.gamma).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    alpha, G1 = 6.0, 1
    smooth, g_s, b_s = zq.smoothquant_factors(Xd, Wd, w.eps, gamma, beta)
    Wq_s, sw_s = zq.quantize_weights_grouped(Wd, w.group_rows, smooth)
    Wq_d, sw_d = zq.quantize_weights_grouped(Wd, G1)
    Wt = zq.pack_outlier_weights(Wd)
    del Wd, smooth
    torch.cuda.synchronize()
    set_bytes = 2 * M * K + N * K * 4 + 2 * M * N + 3 * M * K
    nsets = max(2, math.ceil(args.rotate_mb * 1e6 / set_bytes))
    ws_lin = zq.linear_workspace_bytes(M, K)
    ws_dec = zq.linear_decomp_workspace_bytes(M, K)
    sets = []
    for i in range(nsets):
        sets.append(dict(
            X=Xd if i == 0 else Xd.clone(),
            Wq_s=Wq_s if i == 0 else Wq_s.clone(),
            Wq_d=Wq_d if i == 0 else Wq_d.clone(),
            Wt=Wt if i == 0 else Wt.clone(),
            ws=torch.empty(max(ws_lin, ws_dec), dtype=torch.uint8, device=dev),
            Y=torch.empty((M, N), dtype=torch.float16, device=dev)))

    def smoothquant(i):
        s = sets[i % nsets]
        zq.linear_w8a8(s["X"], s["Wq_s"], sw_s, w.group_rows, w.pre, g_s, b_s, w.eps, None,
                       w.act, workspace=s["ws"], out=s["Y"])

    def decomposed(i):
        s = sets[i % nsets]
        zq.linear_w8a8_decomp(s["X"], s["Wq_d"], sw_d, G1, s["Wt"], alpha, w.pre, gamma, beta,
                              w.eps, None, w.act, workspace=s["ws"], out=s["Y"])

    # The stages, on the buffers zq_linear_w8a8_decomp uses (same workspace layout).
    def parts(s):
        r = lambda v: (v + 255) // 256 * 256  # noqa: E731
        ws = s["ws"]
        o_cols = r(4 * K)
        o_xq = o_cols + r(4 * (K + 1))
        o_sx = o_xq + r(M * K)
        o_xo = o_sx + r(4 * M)
        return (ws[:4 * K].view(torch.int32), ws[o_cols:o_cols + 4 * (K + 1)].view(torch.int32),
                ws[o_xq:o_xq + M * K].view(torch.int8).view(M, K),
                ws[o_sx:o_sx + 4 * M].view(torch.float32),
                ws[o_xo:o_xo + 2 * M * K].view(torch.float16).view(M, K))

    def stage_columns(i):
        s = sets[i % nsets]
        slot, cols, _, _, _ = parts(s)
        zq.outlier_columns(s["X"], alpha, w.pre, gamma, beta, w.eps, out=(slot, cols))

    def stage_prologue(i):
        s = sets[i % nsets]
        slot, _, xq, sx, xo = parts(s)
        zq.ln_quant_decomp(s["X"], slot, w.pre, gamma, beta, w.eps, out=(xq, sx, xo))

    def stage_gemm(i):
        s = sets[i % nsets]
        _, cols, xq, sx, xo = parts(s)
        zq.w8a8_gemm_decomp(xq, sx, s["Wq_d"], sw_d, G1, cols, xo, s["Wt"], None, w.act,
                            out=s["Y"])

    # The int8 GEMM alone on the same codes and weights (no fp16 part): what the
    # fp16 outlier epilogue adds, separated from data-dependent clock effects.
    def stage_gemm_int8(i):
        s = sets[i % nsets]
        _, _, xq, sx, _ = parts(s)
        zq.w8a8_gemm_dequant(xq, sx, s["Wq_d"], sw_d, G1, None, w.act, out=s["Y"])

    res = {}
    for name, fn in (("smoothquant", smoothquant), ("decomposed", decomposed),
                     ("columns", stage_columns), ("prologue", stage_prologue),
                     ("gemm", stage_gemm), ("gemm_int8", stage_gemm_int8)):
        for i in range(nsets):
            fn(i)
        g = graph_of(torch, fn, args.steps)
        time_graph(torch, g)
        res[name] = time_graph(torch, g)[0] / args.steps
        del g
    torch.cuda.synchronize()
    n_out = int(parts(sets[0])[1][0].item())
    ops = 2.0 * M * N * K
    out = {"workload": f"{w.name}: X fp16 [{M} x {K}], W [{N} x {K}], 0.5% channels x100",
           "smoothquant_fused_us": round(res["smoothquant"] * 1e3, 3),
           "smoothquant_TOPS": round(ops / (res["smoothquant"] * 1e-3) / 1e12, 2),
           "decomposed_us": round(res["decomposed"] * 1e3, 3),
           "decomposed_TOPS": round(ops / (res["decomposed"] * 1e-3) / 1e12, 2),
           "decomposed_breakdown_us": {"outlier_columns": round(res["columns"] * 1e3, 3),
                                       "prologue": round(res["prologue"] * 1e3, 3),
                                       "gemm_with_fp16_part": round(res["gemm"] * 1e3, 3),
                                       "same_gemm_without_fp16_part":
                                           round(res["gemm_int8"] * 1e3, 3)},
           "alpha": alpha, "outlier_columns": n_out,
           "weights": {"smoothquant": f"group_rows={w.group_rows}",
                       "decomposed": "group_rows=1 (per output channel) + fp16 [K x N] copy"}}
    del sets, Xd, Wq_s, Wq_d, Wt
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import post_w8a8_quantized_amd as zq
    from zq_workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    zq.library()
    if args.calib_copy_mb > 0:
        calib_copy(torch, args.calib_copy_mb)
        return

    w = WORKLOADS[args.workload]
    decode = w.M <= 32
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    Xd = torch.from_numpy(inp.X).to(dev)
    Wd = torch.from_numpy(inp.W).to(dev)
    gamma = torch.from_numpy(inp.gamma).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)

    # ---- offline (untimed): SmoothQuant fold and group-wise weight quantization
    smooth = None
    if w.smooth:
        smooth, gamma, beta = zq.smoothquant_factors(Xd, Wd, w.eps, gamma, beta)
    Wq, s_w = zq.quantize_weights_grouped(Wd, w.group_rows, smooth)
    del Wd
    if decode:
        # Decode shapes stream the weights once per step: they are re-laid out
        # offline into the packed blocks the weight-streaming kernel reads.
        Wq = zq.pack_weights(Wq)
    torch.cuda.synchronize()
    g_arg = gamma if w.pre == zq.PRE_LAYERNORM else None
    b_arg = beta if w.pre == zq.PRE_LAYERNORM else None

    # ---- rotated sets
    M, N, K, G = w.M, w.N, w.K, w.group_rows
    ws_bytes = zq.linear_workspace_bytes(M, K)
    x_el = 2 if w.x_dtype == "f16" else 4
    set_bytes = M * K * x_el + N * K + M * N * 2 + ws_bytes + 4 * N // G
    nsets = max(2, math.ceil(args.rotate_mb * 1e6 / set_bytes))
    sets = []
    for i in range(nsets):
        sets.append(dict(
            X=Xd if i == 0 else Xd.clone(),
            Wq=Wq if i == 0 else Wq.clone(),
            s_w=s_w if i == 0 else s_w.clone(),
            ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
            Y=torch.empty((M, N), dtype=torch.float16, device=dev),
        ))
    xq_off = 0
    sx_off = (M * K + 255) // 256 * 256

    def layer(i):
        s = sets[i % nsets]
        if decode:
            zq.linear_w8a8_packed(s["X"], s["Wq"], s["s_w"], G, N, w.pre, g_arg, b_arg, w.eps,
                                  bias, w.act, workspace=s["ws"], out=s["Y"])
        else:
            zq.linear_w8a8(s["X"], s["Wq"], s["s_w"], G, w.pre, g_arg, b_arg, w.eps, bias, w.act,
                           workspace=s["ws"], out=s["Y"])

    def prologue(i):
        s = sets[i % nsets]
        xq = s["ws"][xq_off:xq_off + M * K].view(torch.int8).view(M, K)
        sx = s["ws"][sx_off:sx_off + 4 * M].view(torch.float32)
        zq.ln_quant_per_token(s["X"], w.pre, g_arg, b_arg, w.eps, out=(xq, sx))

    def gemm(i):
        s = sets[i % nsets]
        xq = s["ws"][xq_off:xq_off + M * K].view(torch.int8).view(M, K)
        sx = s["ws"][sx_off:sx_off + 4 * M].view(torch.float32)
        if decode:
            zq.w8a8_gemm_dequant_packed(xq, sx, s["Wq"], s["s_w"], G, N, bias, w.act, out=s["Y"])
        else:
            zq.w8a8_gemm_dequant(xq, sx, s["Wq"], s["s_w"], G, bias, w.act, out=s["Y"])

    # eager pass over every set (fills every workspace with valid codes)
    for i in range(nsets):
        layer(i)
    torch.cuda.synchronize()

    # ---- per-kernel averages over graphs of the same launches (HIP events).  They run
    # first: their ~20 ms of work also brings the GPU to the steady state a sustained
    # run sees (a cold GPU runs the first ~10 ms of steps ~10% slower).
    g_pro = graph_of(torch, prologue, args.steps)
    g_gemm = graph_of(torch, gemm, args.steps)
    time_graph(torch, g_pro)
    time_graph(torch, g_gemm)
    pro_ms = time_graph(torch, g_pro)[0] / args.steps
    gemm_ms = time_graph(torch, g_gemm)[0] / args.steps

    # ---- timed layer steps: the W warmup steps are replays of the same K-step graph
    # (ceil(W / K) of them), so the timed replay runs a graph that has already been
    # launched once: a graph's first replay carries one-time costs (~10% of a
    # 400-step replay here) that a sustained run never pays again.
    g_steps = graph_of(torch, layer, args.steps)
    warm_replays = -(-args.warmup // args.steps)
    for _ in range(warm_replays):
        time_graph(torch, g_steps)
    warmup_steps = warm_replays * args.steps
    ms_ev, ms_wall = time_graph(torch, g_steps)
    ms_step = ms_ev / args.steps
    # Spread: further replays of the same K-step graph (outside the timed region).
    reps = np.array([ms_step] + [time_graph(torch, g_steps)[0] / args.steps for _ in range(9)])
    p10, p50, p90 = np.percentile(reps * 1e3, [10, 50, 90])
    spread = {"replays": int(reps.size), "p10_us": round(float(p10), 3),
              "p50_us": round(float(p50), 3), "p90_us": round(float(p90), 3)}
    del g_steps, g_pro, g_gemm
    torch.cuda.synchronize()

    # ---- fusion ablation (prefill shapes): the same layer in the unfused order
    # (op -> fp16 -> quantizer -> int32 GEMM -> dequantizer), same rotated sets;
    # the intermediates share one workspace.
    ablation = None
    if not decode and not args.no_ablation:
        ws_unf = torch.empty(zq.linear_unfused_workspace_bytes(M, N, K), dtype=torch.uint8,
                             device=dev)

        def layer_unfused(i):
            s = sets[i % nsets]
            zq.linear_w8a8_unfused(s["X"], s["Wq"], s["s_w"], G, w.pre, g_arg, b_arg, w.eps,
                                   bias, w.act, workspace=ws_unf, out=s["Y"])

        for i in range(nsets):
            layer_unfused(i)
        g_unf = graph_of(torch, layer_unfused, args.steps)
        time_graph(torch, g_unf)
        unf_ms = time_graph(torch, g_unf)[0] / args.steps
        del g_unf, ws_unf
        torch.cuda.synchronize()
        ablation = {"unfused_layer_step_us": round(unf_ms * 1e3, 3),
                    "fused_layer_step_us": round(ms_step * 1e3, 3),
                    "fusion_speedup": round(unf_ms / ms_step, 3),
                    "unfused_order": "op->fp16, quantize, int8 GEMM->int32, dequantize"}

    ops = 2.0 * M * N * K
    bytes_pro = M * K * x_el + M * K + 4 * M
    bytes_gemm = M * K + 4 * M + N * K + 4 * (N // G) + (4 * N if bias is not None else 0) + 2 * M * N
    bytes_layer = bytes_pro + bytes_gemm
    gemm_kernel = "gemm_skinny" if decode else "gemm_tiled"
    src_hash = kernel_source_hash([f"{gemm_kernel}.hip", "zq_device.h"])
    traffic = read_traffic(gemm_kernel, w.name, src_hash)

    if decode:
        value = bytes_layer / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        g_ach = bytes_gemm / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(g_ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(g_ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel": gemm_kernel, "avg_launch_us": round(gemm_ms * 1e3, 3),
                    "algorithmic_bytes_per_launch": bytes_gemm}
    else:
        value = ops / (ms_step * 1e-3) / 1e12
        unit = "TOPS"
        g_ach = ops / (gemm_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(g_ach, 1), "peak": PEAK_INT8_TOPS,
                    "unit": "TOP/s", "frac": round(g_ach / PEAK_INT8_TOPS, 4), "traffic": traffic,
                    "kernel": gemm_kernel, "avg_launch_us": round(gemm_ms * 1e3, 3),
                    "algorithmic_ops_per_launch": ops, "algorithmic_bytes_per_launch": bytes_gemm}
    # counted HBM bytes over the bytes the kernel must move (re-reads, partial lines)
    roofline["traffic_over_algorithmic"] = (round(traffic / bytes_gemm, 3) if traffic
                                            else None)

    # ---- chained FFN block (BERT FFN-up shape): FFN-up then FFN-down (W2 [K x N] drawn
    # like W), as one zq_ffn_w8a8 call against two zq_linear_w8a8 calls
    ffn = None
    if w.name == "bert_ffn_up" and not args.no_ffn:
        g2 = torch.Generator(device="cpu").manual_seed(1)
        W2 = (0.02 * torch.randn((K, N), generator=g2, dtype=torch.float32)).to(dev)
        W2q, s_w2 = zq.quantize_weights_grouped(W2, G)
        b2 = (0.01 * torch.randn((K,), generator=g2, dtype=torch.float32)).to(dev)
        del W2
        H = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws_ffn = torch.empty(zq.ffn_workspace_bytes(M, K, N), dtype=torch.uint8, device=dev)
        ws_lin2 = torch.empty(zq.linear_workspace_bytes(M, N), dtype=torch.uint8, device=dev)
        Yb = [torch.empty((M, K), dtype=torch.float16, device=dev) for _ in range(nsets)]

        def block_chained(i):
            s = sets[i % nsets]
            zq.ffn_w8a8(s["X"], s["Wq"], s["s_w"], G, W2q, s_w2, G, g_arg, b_arg, w.eps, bias, b2,
                        workspace=ws_ffn, out=Yb[i % nsets])

        def block_two_calls(i):
            s = sets[i % nsets]
            zq.linear_w8a8(s["X"], s["Wq"], s["s_w"], G, w.pre, g_arg, b_arg, w.eps, bias, w.act,
                           workspace=s["ws"], out=H)
            zq.linear_w8a8(H, W2q, s_w2, G, zq.PRE_NONE, None, None, w.eps, b2, zq.ACT_NONE,
                           workspace=ws_lin2, out=Yb[i % nsets])

        res = {}
        for name, fn in (("chained", block_chained), ("two_calls", block_two_calls)):
            for i in range(nsets):
                fn(i)
            g = graph_of(torch, fn, args.steps)
            time_graph(torch, g)
            res[name] = time_graph(torch, g)[0] / args.steps
            del g
        torch.cuda.synchronize()
        ops_blk = 2.0 * 2.0 * M * N * K
        ffn = {"block": f"FFN {K}->{N}->{K}, {M} tokens",
               "chained_us": round(res["chained"] * 1e3, 3),
               "two_calls_us": round(res["two_calls"] * 1e3, 3),
               "chained_TOPS": round(ops_blk / (res["chained"] * 1e-3) / 1e12, 2)}
        del ws_ffn, ws_lin2, Yb, H, W2q, s_w2, b2

    # ---- FP8 variant of the same layer (E4M3 codes, power-of-two scales), weights
    # quantized offline (and packed at decode shapes), same rotated inputs
    fp8 = None
    if not args.no_fp8:
        Wd8 = torch.from_numpy(inp.W).to(dev)
        W8, s_w8 = zq.quantize_weights_grouped_fp8(Wd8, G, smooth)
        del Wd8
        if decode:
            W8 = zq.pack_weights(W8)
        W8s = [W8] + [W8.clone() for _ in range(nsets - 1)]   # rotated like the int8 weights
        Y8 = torch.empty((M, N), dtype=torch.float16, device=dev)

        def layer_fp8(i):
            s = sets[i % nsets]
            zq.linear_w8a8_fp8(s["X"], W8s[i % nsets], s_w8, G, w.pre, g_arg, b_arg, w.eps, bias,
                               w.act, workspace=s["ws"], out=Y8, N=N, packed=decode)

        for i in range(nsets):
            layer_fp8(i)
        g8 = graph_of(torch, layer_fp8, args.steps)
        time_graph(torch, g8)
        ms8 = time_graph(torch, g8)[0] / args.steps
        del g8, W8, W8s, Y8
        torch.cuda.synchronize()
        fp8 = {"layer_step_us": round(ms8 * 1e3, 3),
               "value": round((bytes_layer / (ms8 * 1e-3) / 1e9) if decode
                              else (ops / (ms8 * 1e-3) / 1e12), 2),
               "unit": "GB/s" if decode else "TOPS"}

    # ---- the outlier workload (X fp16 [4096 x 5120], 0.5% of channels x100, LayerNorm;
    # W [13824 x 5120]) under its two treatments: the SmoothQuant fold with the fused
    # W8A8 layer (G = 128), and the mixed-precision decomposition (outlier columns in
    # fp16, per-output-channel int8 weights, alpha = 6).  Each on its own rotated sets.
    decomp = None
    if not args.no_decomp:
        decomp = outlier_leg(torch, zq, WORKLOADS["outlier_smooth"], make_inputs, args, dev)

    # ---- achievable HBM bandwidth for context: a 1 GiB device-to-device copy
    # (torch's copy kernel; read + write bytes over the HIP-event time of 5 copies)
    hbm_ref = None
    if not args.no_copy_reference:
        torch.cuda.synchronize()
        nb = 1 << 30
        ca = torch.ones(nb, dtype=torch.uint8, device=dev)
        cb = torch.empty_like(ca)
        cb.copy_(ca)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            cb.copy_(ca)
        e1.record()
        torch.cuda.synchronize()
        ms_copy = e0.elapsed_time(e1) / 5
        hbm_ref = {"copy_GBps": round(2 * nb / (ms_copy * 1e-3) / 1e9, 1),
                   "bytes_moved": 2 * nb, "what": "1 GiB device copy (read + write), context only"}
        del ca, cb

    # ---- CPU oracle on the host cores (a reported baseline, not the target)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        Wq_h, sw_h = ref.quantize_groups(
            ref.fold_weights(inp.W, smooth.cpu().numpy()) if smooth is not None else inp.W, G)
        g_h = gamma.cpu().numpy() if w.pre == 1 else None
        b_h = beta.cpu().numpy() if w.pre == 1 else None
        rows = np.arange(M, dtype=np.int64)

        def oracle_passes(seconds):
            passes, t0 = 0, time.perf_counter()
            while True:
                ref.linear_rows(inp.X, w.pre, g_h, b_h, w.eps, Wq_h, sw_h, G, inp.bias, w.act,
                                rows)
                passes += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    return passes, el

        def rate(per):
            return round((bytes_layer / per / 1e9) if decode else (ops / per / 1e12), 4)

        cores = ref.max_threads()
        passes, el = oracle_passes(args.cpu_seconds)
        per = el / passes
        cpu = {"value": rate(per), "unit": unit, "cores": cores, "kind": "oracle",
               "sample": f"all {M} tokens of the workload (prologue + int GEMM + epilogue), "
                         f"{passes} passes, {per:.3f} s each, {el:.1f} s wall on {cores} threads"}
        if decode:
            # the few-token shapes also on one core (at least one pass, about 3 s)
            ref.set_threads(1)
            passes1, el1 = oracle_passes(3.0)
            ref.set_threads(cores)
            cpu["one_thread"] = {"value": rate(el1 / passes1), "unit": unit,
                                 "sample": f"{passes1} passes, {el1 / passes1:.3f} s each"}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup_steps,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "K": K, "N": N, "group_rows": G,
                   "x_dtype": w.x_dtype, "pre": PRE_NAMES[w.pre], "act": ACT_NAMES[w.act],
                   "bias": bias is not None, "smoothquant": w.smooth,
                   "weights": "packed 32x512 blocks" if decode else "row-major",
                   "rotated_sets": nsets, "graph_steps": args.steps},
        "frac_of_peak": round(value / (PEAK_HBM_GBS if decode else PEAK_INT8_TOPS), 4),
        "breakdown_us": {"layer_step": round(ms_step * 1e3, 3), "prologue": round(pro_ms * 1e3, 3),
                         "gemm": round(gemm_ms * 1e3, 3),
                         "prologue_GBps": round(bytes_pro / (pro_ms * 1e-3) / 1e9, 1),
                         "timed_region_wall_ms": round(ms_wall, 3),
                         "layer_step_spread": spread},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_copy_reference": hbm_ref,
        "ablation": ablation,
        "ffn_block": ffn,
        "fp8_variant": fp8,
        "outlier_decomposition": decomp,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
