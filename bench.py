"""Benchmark of the W8A8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the per-token hot path over one batch: the fused
LayerNorm/GeLU + per-token quantization kernel, then the int8 MFMA GEMM with
the fused dequant (+bias, +GeLU) epilogue, through zq_linear_w8a8.  Weights
are quantized offline (by the library) before timing, as the method
prescribes.  Inputs are seeded synthetic data resident in HBM; several
independent input/weight/output sets are rotated so that the 256 MB
Infinity Cache cannot serve a step from the previous one.

The headline workload (default: the largest, X fp16 [4096 x 5120] with 0.5%
outlier channels, SmoothQuant fold, W [13824 x 5120]) is timed with every
leg: the dominant kernel's roofline, the fusion ablation, the FP8 variant and
the CPU oracle on the host cores.  The other workloads (BERT FFN-up, GPT QKV,
decode FFN-down) follow as extra keys, each with its layer time, fraction of
peak and its dominant kernel's roofline, and the outlier workload is timed
again under the mixed-precision decomposition.  For the prefill workloads the
vendor library's int8 GEMM (torch._int_mm, hipBLASLt) is timed on the same
codes for context (library_leg).

The steps are captured in a HIP graph (on torch's stream, which is the
stream the library launches on) so that host-side call overhead does not
leave the GPU idle between layers; the timed region is one replay of a graph
of exactly K steps, bracketed by device synchronisations.  The prologue's and
the GEMM's average launch durations (the roofline's) come from K more steps
with HIP events between the two kernels, queued behind replays of that graph
so that they run in the same back-to-back state (kernel_times).

Printed: ONE JSON line.
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
PEAK_CLOCK_MHZ = 2400.0     # the graphics clock the published MFMA peak assumes
PRE_NAMES = {0: "none", 1: "layernorm", 2: "gelu"}
ACT_NAMES = {0: "none", 1: "gelu"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="outlier_smooth",
                    help="the headline workload (default: the largest, the outlier layer "
                         "with the SmoothQuant fold)")
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
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads (BERT FFN-up, GPT QKV, decode FFN-down)")
    ap.add_argument("--no-clock-sample", action="store_true",
                    help="skip the untimed back-to-back steps (2 s) before each workload's "
                         "warmup, during which amd-smi samples the GPU clock and power; for "
                         "profiler runs")
    ap.add_argument("--no-copy-reference", action="store_true",
                    help="skip the 1 GiB device-copy bandwidth reference")
    ap.add_argument("--no-library-reference", action="store_true",
                    help="skip the vendor int8 GEMM (torch._int_mm, hipBLASLt) comparison "
                         "(prefill workloads)")
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


def settled_ms(torch, g, steps, args):
    """Milliseconds per step of one replay of graph g (`steps` steps), after the
    warmup replays and, unless --no-clock-sample, 0.3 s of back-to-back replays
    (the GPU runs slower for a while after any idle time; settle_and_sample)."""
    if not args.no_clock_sample:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            g.replay()
            torch.cuda.synchronize()
    for _ in range(-(-args.warmup // steps)):
        time_graph(torch, g)
    return time_graph(torch, g)[0] / steps


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


def settle_and_sample(torch, g, seconds=2.0, sample=True):
    """Replays graph g (K layer steps) back to back for about `seconds`, right
    before the warmup and timed replays, so that those run at the clock and
    power the GPU sustains under this load: after any idle time the GPU comes
    back slower (measured on the headline layer: 295 us per step back to back,
    ~305 us with 2 ms of host idle before each replay, ~340 us with 50 ms, and
    ~20 ms of work to recover).  With `sample`, amd-smi samples the socket
    power and the per-XCD graphics clocks meanwhile; returns their medians
    (None without sampling or amd-smi, or under a profiler, whose preloaded
    library would also attach to amd-smi's process).  Untimed."""
    import shutil
    import statistics
    import subprocess
    import threading
    cmd = None
    profiled = any(k.startswith("ROCPROF") for k in os.environ) or \
        "rocprofiler" in os.environ.get("LD_PRELOAD", "")
    exe = None if (profiled or not sample) else shutil.which("amd-smi")
    if exe is not None:
        # amd-smi is a Python script: run it with this interpreter as a child
        # process (no `env` hop that would exec a second program).
        exe = os.path.realpath(exe)
        with open(exe, "rb") as fh:
            first = fh.readline()
        cmd = [sys.executable, exe] if first.startswith(b"#!") and b"python" in first else [exe]
    rows, stop = [], [False]

    def sampler():
        while not stop[0]:
            try:
                r = subprocess.run(cmd + ["metric", "-p", "-c", "--csv"], capture_output=True,
                                   text=True, timeout=10)
            except (subprocess.TimeoutExpired, OSError):
                return
            lines = [ln for ln in r.stdout.strip().splitlines() if ln.strip()]
            if len(lines) >= 2:
                rows.append(dict(zip(lines[0].split(","), lines[-1].split(","))))
            time.sleep(0.2)

    th = threading.Thread(target=sampler, daemon=True) if cmd else None
    torch.cuda.synchronize()
    if th:
        th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        g.replay()
        torch.cuda.synchronize()
    stop[0] = True
    # keep the GPU busy until the sampler's last amd-smi call has returned (each
    # call is bounded), so that no idle time separates this from the warmup replays
    while th is not None and th.is_alive() and time.perf_counter() - t0 < seconds + 15.0:
        g.replay()
        torch.cuda.synchronize()
    if th:
        th.join(timeout=15.0)
    if not cmd:
        return None
    rows = rows[2:-1] if len(rows) > 4 else rows   # drop the ramp at both ends

    def med(keys):
        vals = []
        for r in rows:
            for k in keys:
                try:
                    vals.append(float(r[k]))
                except (KeyError, ValueError):
                    pass
        return round(statistics.median(vals), 1) if vals else None

    clk_keys = [k for k in (rows[0] if rows else {}) if k.startswith("gfx_") and k.endswith("_clk")
                and "min" not in k and "max" not in k]
    return {"samples": len(rows), "socket_power_W": med(["socket_power"]),
            "gfx_clock_MHz": med(clk_keys),
            "what": "amd-smi during 2 s of back-to-back replays of the layer-step graph "
                    "before the warmup and timed replays (untimed)"}


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
        res[name] = settled_ms(torch, g, args.steps, args)
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


def prepare(torch, zq, w, make_inputs, args, dev):
    """Offline steps (untimed) and the rotated input sets of one workload."""
    inp = make_inputs(w)
    decode = w.M <= 32
    Xd = torch.from_numpy(inp.X).to(dev)
    Wd = torch.from_numpy(inp.W).to(dev)
    gamma = torch.from_numpy(inp.gamma).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    # ---- offline: SmoothQuant fold and group-wise weight quantization
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
    return dict(w=w, inp=inp, decode=decode, gamma=gamma, beta=beta, bias=bias, smooth=smooth,
                g_arg=gamma if w.pre == zq.PRE_LAYERNORM else None,
                b_arg=beta if w.pre == zq.PRE_LAYERNORM else None,
                sets=sets, nsets=nsets, x_el=x_el)


def kernel_times(torch, g_steps, ms_step, prologue, gemm, steps):
    """Average launch durations of the prologue and the GEMM as they run inside
    layer steps.  ROCm's PyTorch records no timing events inside a captured
    graph, so the K steps run eagerly, the prologue and the GEMM as the two
    boundary calls with HIP events on the launch stream before, between and
    after them.  They are queued behind replays of the timed graph (at least
    ~25 ms of GPU work, far more than the host needs to queue the K steps,
    with Python's garbage collector held off meanwhile), so the GPU never
    waits for the host and the kernels run in the same back-to-back state as
    in the timed replay.  Returns (prologue ms, GEMM ms, idle fraction of the
    steps' span, [p10, p50, p90] of the GEMM's per-step durations in us)."""
    import gc
    import numpy as np
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    lead = max(1, -(-25.0 // (ms_step * steps)))
    torch.cuda.synchronize()
    gc_was_on = gc.isenabled()
    gc.disable()
    try:
        for _ in range(int(lead)):
            g_steps.replay()
        for i in range(steps):
            a, b, c = ev[i]
            a.record()
            prologue(i)
            b.record()
            gemm(i)
            c.record()
    finally:
        if gc_was_on:
            gc.enable()
    torch.cuda.synchronize()
    pro = np.array([a.elapsed_time(b) for a, b, _ in ev])
    gem = np.array([b.elapsed_time(c) for _, b, c in ev])
    span = ev[0][0].elapsed_time(ev[-1][2])
    gap = max(0.0, 1.0 - float(pro.sum() + gem.sum()) / span) if span > 0 else 0.0
    spread = [round(float(np.percentile(gem, q)) * 1e3, 3) for q in (10, 50, 90)]
    return float(pro.mean()), float(gem.mean()), gap, spread


def time_layer(torch, zq, st, args, sample=False):
    """HIP-event time of K whole layer steps (one replay of a K-step graph after
    the warmup replays), the prologue's and the GEMM's average launch durations
    in the same steps (kernel_times), and the dominant kernel's roofline."""
    import numpy as np
    w, sets, nsets, decode = st["w"], st["sets"], st["nsets"], st["decode"]
    M, N, K, G = w.M, w.N, w.K, w.group_rows
    g_arg, b_arg, bias = st["g_arg"], st["b_arg"], st["bias"]
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
    # timed layer steps: the W warmup steps are replays of the same K-step graph
    # (ceil(W / K) of them), so the timed replay runs a graph that has already been
    # launched once (a graph's first replay carries one-time costs).
    g_steps = graph_of(torch, layer, args.steps)
    clock_power = None
    if not args.no_clock_sample:
        clock_power = settle_and_sample(torch, g_steps, 2.0 if sample else 0.5, sample)
    warm_replays = -(-args.warmup // args.steps)
    for _ in range(warm_replays):
        time_graph(torch, g_steps)
    ms_ev, ms_wall = time_graph(torch, g_steps)
    ms_step = ms_ev / args.steps
    reps = np.array([ms_step] + [time_graph(torch, g_steps)[0] / args.steps for _ in range(9)])
    p10, p50, p90 = np.percentile(reps * 1e3, [10, 50, 90])
    pro_ms, gemm_ms, gap, gemm_spread = kernel_times(torch, g_steps, ms_step, prologue, gemm,
                                                     args.steps)
    del g_steps
    torch.cuda.synchronize()

    ops = 2.0 * M * N * K
    bytes_pro = M * K * st["x_el"] + M * K + 4 * M
    bytes_gemm = (M * K + 4 * M + N * K + 4 * (N // G) + (4 * N if bias is not None else 0)
                  + 2 * M * N)
    bytes_layer = bytes_pro + bytes_gemm
    gemm_kernel = "gemm_skinny" if decode else "gemm_tiled"
    src_hash = kernel_source_hash([f"{gemm_kernel}.hip", "zq_device.h"])
    traffic = read_traffic(gemm_kernel, w.name, src_hash)
    if decode:
        value, unit, peak = bytes_layer / (ms_step * 1e-3) / 1e9, "GB/s", PEAK_HBM_GBS
        g_ach = bytes_gemm / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(g_ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(g_ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel": gemm_kernel, "avg_launch_us": round(gemm_ms * 1e3, 3),
                    "algorithmic_bytes_per_launch": bytes_gemm}
    else:
        value, unit, peak = ops / (ms_step * 1e-3) / 1e12, "TOPS", PEAK_INT8_TOPS
        g_ach = ops / (gemm_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(g_ach, 1), "peak": PEAK_INT8_TOPS,
                    "unit": "TOP/s", "frac": round(g_ach / PEAK_INT8_TOPS, 4), "traffic": traffic,
                    "kernel": gemm_kernel, "avg_launch_us": round(gemm_ms * 1e3, 3),
                    "algorithmic_ops_per_launch": ops, "algorithmic_bytes_per_launch": bytes_gemm}
    # counted HBM bytes over the bytes the kernel must move (re-reads, partial lines)
    roofline["traffic_over_algorithmic"] = (round(traffic / bytes_gemm, 3) if traffic else None)
    roofline["launch_timing"] = ("HIP events around each launch in K eager layer steps queued "
                                 "behind replays of the timed graph; GPU idle between the "
                                 f"step's kernels: {gap * 100:.2f}% of the steps' span")
    roofline["launch_us_p10_p50_p90"] = gemm_spread
    # Context for a compute-bound kernel: the published peak assumes 2.4 GHz; the
    # same peak scaled to the graphics clock amd-smi read during back-to-back
    # steps of this layer (the chip holds its power limit there).  `frac` above
    # stays against the published peak.
    clk = (clock_power or {}).get("gfx_clock_MHz")
    if not decode and clk:
        peak_clk = PEAK_INT8_TOPS * clk / PEAK_CLOCK_MHZ
        roofline["at_sampled_clock"] = {"gfx_clock_MHz": clk, "peak": round(peak_clk, 1),
                                        "frac": round(g_ach / peak_clk, 4)}
    return dict(ms_step=ms_step, ms_wall=ms_wall, pro_ms=pro_ms, gemm_ms=gemm_ms, value=value,
                nsets=nsets, clock_power=clock_power,
                unit=unit, peak=peak, ops=ops, bytes_pro=bytes_pro, bytes_gemm=bytes_gemm,
                bytes_layer=bytes_layer, roofline=roofline,
                spread={"replays": int(reps.size), "p10_us": round(float(p10), 3),
                        "p50_us": round(float(p50), 3), "p90_us": round(float(p90), 3)})


def fp8_leg(torch, zq, st, t, args, dev):
    """The FP8 variant of the same layer (E4M3 codes, power-of-two scales), weights
    quantized offline (and packed at decode shapes), same rotated inputs."""
    w, sets, nsets, decode = st["w"], st["sets"], st["nsets"], st["decode"]
    M, N, G = w.M, w.N, w.group_rows
    Wd8 = torch.from_numpy(st["inp"].W).to(dev)
    W8, s_w8 = zq.quantize_weights_grouped_fp8(Wd8, G, st["smooth"])
    del Wd8
    if decode:
        W8 = zq.pack_weights(W8)
    W8s = [W8] + [W8.clone() for _ in range(nsets - 1)]   # rotated like the int8 weights
    Y8 = torch.empty((M, N), dtype=torch.float16, device=dev)

    def layer_fp8(i):
        s = sets[i % nsets]
        zq.linear_w8a8_fp8(s["X"], W8s[i % nsets], s_w8, G, w.pre, st["g_arg"], st["b_arg"],
                           w.eps, st["bias"], w.act, workspace=s["ws"], out=Y8, N=N,
                           packed=decode)

    for i in range(nsets):
        layer_fp8(i)
    g8 = graph_of(torch, layer_fp8, args.steps)
    ms8 = settled_ms(torch, g8, args.steps, args)
    del g8, W8, W8s, Y8
    torch.cuda.synchronize()
    return {"layer_step_us": round(ms8 * 1e3, 3),
            "value": round((t["bytes_layer"] / (ms8 * 1e-3) / 1e9) if decode
                           else (t["ops"] / (ms8 * 1e-3) / 1e12), 2),
            "unit": "GB/s" if decode else "TOPS"}


def library_leg(torch, zq, st, args, dev):
    """Context, not the product path: the vendor library's int8 GEMM (torch._int_mm,
    which runs hipBLASLt) on the layer's own codes and weights, int32 out, against
    this library's GEMM on the same operands in its int32 test mode and with its
    fused fp16 dequant epilogue.  Each is timed over `steps` eager launches queued
    back to back (HIP events around them, rotated sets, after 0.3 s of untimed
    launches), three rounds in alternation, median per launch.  Also checks that
    the two int32 products agree bit for bit."""
    w, sets, nsets = st["w"], st["sets"], st["nsets"]
    M, N, K, G = w.M, w.N, w.K, w.group_rows
    codes = [zq.ln_quant_per_token(s["X"], w.pre, st["g_arg"], st["b_arg"], w.eps) for s in sets]
    y32 = torch.empty((M, N), dtype=torch.int32, device=dev)
    y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()
    equal = bool(torch.equal(torch._int_mm(codes[0][0], sets[0]["Wq"].t()),
                             zq.w8a8_gemm_dequant(codes[0][0], None, sets[0]["Wq"], None, G,
                                                  out_dtype=torch.int32, out=y32)))

    def lib(i):
        torch._int_mm(codes[i % nsets][0], sets[i % nsets]["Wq"].t())

    def ours32(i):
        zq.w8a8_gemm_dequant(codes[i % nsets][0], None, sets[i % nsets]["Wq"], None, G,
                             out_dtype=torch.int32, out=y32)

    def ours16(i):
        Xq, sx = codes[i % nsets]
        zq.w8a8_gemm_dequant(Xq, sx, sets[i % nsets]["Wq"], sets[i % nsets]["s_w"], G,
                             st["bias"], w.act, out=y16)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            for i in range(nsets):
                fn(i)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    us = {"lib": [], "i32": [], "f16": []}
    for _ in range(3):
        us["lib"].append(timed(lib))
        us["i32"].append(timed(ours32))
        us["f16"].append(timed(ours16))
    med = {k: sorted(v)[1] for k, v in us.items()}
    ops = 2.0 * M * N * K
    del codes, y32, y16
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"what": "torch._int_mm (hipBLASLt) int8 x int8 -> int32 on the layer's codes and "
                    "weights vs this library's GEMM on the same operands; eager launches, "
                    "context only",
            "library_int32_us": round(med["lib"], 2),
            "library_int32_TOPS": round(ops / (med["lib"] * 1e-6) / 1e12, 1),
            "ours_int32_us": round(med["i32"], 2),
            "ours_int32_TOPS": round(ops / (med["i32"] * 1e-6) / 1e12, 1),
            "ours_fp16_dequant_us": round(med["f16"], 2),
            "ours_int32_over_library_time": round(med["i32"] / med["lib"], 3),
            "int32_results_equal": equal}


def guarded_library_leg(torch, zq, st, args, dev):
    """library_leg, or the reason it could not run (the vendor call is context
    only: a torch build without it, or one that rejects the shape, must not
    cost the benchmark line)."""
    try:
        return library_leg(torch, zq, st, args, dev)
    except (RuntimeError, AttributeError, TypeError) as e:
        torch.cuda.synchronize()
        return {"error": f"{type(e).__name__}: {e}"[:300]}


def ablation_leg(torch, zq, st, t, args, dev):
    """The same layer in the unfused order (op -> fp16 -> quantizer -> int32 GEMM
    -> dequantizer), same rotated sets; the intermediates share one workspace."""
    w, sets, nsets = st["w"], st["sets"], st["nsets"]
    M, N, K, G = w.M, w.N, w.K, w.group_rows
    ws_unf = torch.empty(zq.linear_unfused_workspace_bytes(M, N, K), dtype=torch.uint8,
                         device=dev)

    def layer_unfused(i):
        s = sets[i % nsets]
        zq.linear_w8a8_unfused(s["X"], s["Wq"], s["s_w"], G, w.pre, st["g_arg"], st["b_arg"],
                               w.eps, st["bias"], w.act, workspace=ws_unf, out=s["Y"])

    for i in range(nsets):
        layer_unfused(i)
    g_unf = graph_of(torch, layer_unfused, args.steps)
    unf_ms = settled_ms(torch, g_unf, args.steps, args)
    del g_unf, ws_unf
    torch.cuda.synchronize()
    return {"unfused_layer_step_us": round(unf_ms * 1e3, 3),
            "fused_layer_step_us": round(t["ms_step"] * 1e3, 3),
            "fusion_speedup": round(unf_ms / t["ms_step"], 3),
            "unfused_order": "op->fp16, quantize, int8 GEMM->int32, dequantize"}


def ffn_leg(torch, zq, st, args, dev):
    """Chained FFN block at the BERT FFN-up shape: FFN-up then FFN-down (W2 [K x N]
    drawn like W), as one zq_ffn_w8a8 call against two zq_linear_w8a8 calls, and
    each half alone."""
    w, sets, nsets = st["w"], st["sets"], st["nsets"]
    M, N, K, G = w.M, w.N, w.K, w.group_rows
    g_arg, b_arg, bias = st["g_arg"], st["b_arg"], st["bias"]
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

    def up_only(i):
        s = sets[i % nsets]
        zq.linear_w8a8(s["X"], s["Wq"], s["s_w"], G, w.pre, g_arg, b_arg, w.eps, bias, w.act,
                       workspace=s["ws"], out=H)

    def down_only(i):
        zq.linear_w8a8(H, W2q, s_w2, G, zq.PRE_NONE, None, None, w.eps, b2, zq.ACT_NONE,
                       workspace=ws_lin2, out=Yb[i % nsets])

    def block_two_calls(i):
        up_only(i)
        down_only(i)

    res = {}
    for name, fn in (("chained", block_chained), ("two_calls", block_two_calls),
                     ("up", up_only), ("down", down_only)):
        for i in range(nsets):
            fn(i)
        g = graph_of(torch, fn, args.steps)
        res[name] = settled_ms(torch, g, args.steps, args)
        del g
    torch.cuda.synchronize()
    ops_blk = 2.0 * 2.0 * M * N * K
    return {"block": f"FFN {K}->{N}->{K}, {M} tokens",
            "chained_us": round(res["chained"] * 1e3, 3),
            "two_calls_us": round(res["two_calls"] * 1e3, 3),
            "ffn_up_layer_us": round(res["up"] * 1e3, 3),
            "ffn_down_layer_us": round(res["down"] * 1e3, 3),
            "chained_TOPS": round(ops_blk / (res["chained"] * 1e-3) / 1e12, 2)}


def cpu_model():
    """The host CPU's model name (Linux), for the baseline's context."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_leg(zq, st, t, args, seconds=None):
    """The oracle on the host cores over all tokens of the workload, repeated
    until `seconds` (default args.cpu_seconds) of wall time have passed (a
    reported baseline); for few-token workloads also on one thread."""
    import numpy as np
    from oracle import ref
    w, inp, decode = st["w"], st["inp"], st["decode"]
    G = w.group_rows
    smooth = st["smooth"]
    Wq_h, sw_h = ref.quantize_groups(
        ref.fold_weights(inp.W, smooth.cpu().numpy()) if smooth is not None else inp.W, G)
    g_h = st["gamma"].cpu().numpy() if w.pre == 1 else None
    b_h = st["beta"].cpu().numpy() if w.pre == 1 else None
    rows = np.arange(w.M, dtype=np.int64)

    def oracle_passes(seconds):
        passes, t0 = 0, time.perf_counter()
        while True:
            ref.linear_rows(inp.X, w.pre, g_h, b_h, w.eps, Wq_h, sw_h, G, inp.bias, w.act, rows)
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return passes, el

    def rate(per):
        return round((t["bytes_layer"] / per / 1e9) if decode else (t["ops"] / per / 1e12), 4)

    cores = ref.max_threads()
    passes, el = oracle_passes(args.cpu_seconds if seconds is None else seconds)
    per = el / passes
    cpu = {"value": rate(per), "unit": t["unit"], "cores": cores, "kind": "oracle",
           "sample": f"all {w.M} tokens of the workload (prologue + int GEMM + epilogue), "
                     f"{passes} passes, {per:.3f} s each, {el:.1f} s wall on {cores} threads",
           "host": {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count()}}
    if decode:
        ref.set_threads(1)
        passes1, el1 = oracle_passes(3.0)
        ref.set_threads(cores)
        cpu["one_thread"] = {"value": rate(el1 / passes1), "unit": t["unit"],
                             "sample": f"{passes1} passes, {el1 / passes1:.3f} s each"}
    return cpu


def min_traffic(w, t):
    """At decode shapes: the layer's rate over the bytes a single kernel would
    move (X in, Y out, the weights, their scales and bias), i.e. without the
    codes' and scales' round trip between the prologue and the GEMM."""
    if t["unit"] != "GB/s":
        return {}
    min_bytes = t["bytes_layer"] - 2 * (w.M * w.K + 4 * w.M)
    rate = min_bytes / (t["ms_step"] * 1e-3) / 1e9
    return {"min_traffic_bytes": min_bytes, "min_traffic_GBps": round(rate, 1),
            "min_traffic_frac_of_hbm": round(rate / PEAK_HBM_GBS, 4)}


def summary(w, t):
    """One workload's figures as an extra key of the JSON line."""
    r = t["roofline"]
    out = {"layer_step_us": round(t["ms_step"] * 1e3, 3), "layer_step_spread": t["spread"],
           "value": round(t["value"], 2),
           "unit": t["unit"], "frac_of_peak": round(t["value"] / t["peak"], 4),
           "prologue_us": round(t["pro_ms"] * 1e3, 3),
           "prologue_GBps": round(t["bytes_pro"] / (t["pro_ms"] * 1e-3) / 1e9, 1),
           "prologue_frac_of_hbm": round(t["bytes_pro"] / (t["pro_ms"] * 1e-3) / 1e9
                                         / PEAK_HBM_GBS, 4),
           "gemm_us": round(t["gemm_ms"] * 1e3, 3), "roofline": r,
           "clock_power": t["clock_power"],
           **min_traffic(w, t),
           "config": {"M": w.M, "K": w.K, "N": w.N, "group_rows": w.group_rows,
                      "x_dtype": w.x_dtype, "pre": PRE_NAMES[w.pre], "act": ACT_NAMES[w.act],
                      "bias": w.has_bias, "smoothquant": w.smooth}}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import post_w8a8_quantized_amd as zq
    from zq_workloads import WORKLOAD_ORDER, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    zq.library()
    if args.calib_copy_mb > 0:
        calib_copy(torch, args.calib_copy_mb)
        return
    dev = torch.device("cuda:0")

    # ---- the headline workload, with every leg
    w = WORKLOADS[args.workload]
    st = prepare(torch, zq, w, make_inputs, args, dev)
    t = time_layer(torch, zq, st, args, sample=not args.no_clock_sample)
    ablation = None
    if not st["decode"] and not args.no_ablation:
        ablation = ablation_leg(torch, zq, st, t, args, dev)
    ffn = None
    if w.name == "bert_ffn_up" and not args.no_ffn:
        ffn = ffn_leg(torch, zq, st, args, dev)
    fp8 = None if args.no_fp8 else fp8_leg(torch, zq, st, t, args, dev)
    libref = None
    if not st["decode"] and not args.no_library_reference:
        libref = guarded_library_leg(torch, zq, st, args, dev)
    cpu = None if args.no_cpu_baseline else cpu_leg(zq, st, t, args)
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ---- the outlier workload under the mixed-precision decomposition (its own sets)
    decomp = None
    if not args.no_decomp:
        decomp = outlier_leg(torch, zq, WORKLOADS["outlier_smooth"], make_inputs, args, dev)
        torch.cuda.empty_cache()

    # ---- the other workloads: layer, prologue, GEMM, roofline, FP8 (and the FFN
    # block at the BERT FFN-up shape); each on its own rotated sets
    others = {}
    if not args.no_others:
        for name in WORKLOAD_ORDER:
            if name == w.name or name == "tiny":
                continue
            wo = WORKLOADS[name]
            so = prepare(torch, zq, wo, make_inputs, args, dev)
            to = time_layer(torch, zq, so, args, sample=not args.no_clock_sample)
            others[name] = summary(wo, to)
            if not args.no_fp8:
                others[name]["fp8_variant"] = fp8_leg(torch, zq, so, to, args, dev)
            if not so["decode"] and not args.no_library_reference:
                others[name]["library_reference"] = guarded_library_leg(torch, zq, so, args, dev)
            if name == "bert_ffn_up" and not args.no_ffn:
                others[name]["ffn_block"] = ffn_leg(torch, zq, so, args, dev)
            if so["decode"] and not args.no_cpu_baseline:
                others[name]["cpu_baseline"] = cpu_leg(zq, so, to, args, seconds=4.0)
            del so
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    # ---- achievable HBM bandwidth for context: a 1 GiB device-to-device copy
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

    warmup_steps = -(-args.warmup // args.steps) * args.steps
    out = {
        "metric": METRIC,
        "value": round(t["value"], 2),
        "unit": t["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup_steps,
        "ms_per_step": round(t["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "group_rows": w.group_rows,
                   "x_dtype": w.x_dtype, "pre": PRE_NAMES[w.pre], "act": ACT_NAMES[w.act],
                   "bias": w.has_bias, "smoothquant": w.smooth,
                   "weights": "packed 32x512 blocks" if st_decode(w) else "row-major",
                   "rotated_sets": t.get("nsets"), "graph_steps": args.steps},
        "frac_of_peak": round(t["value"] / t["peak"], 4),
        **min_traffic(w, t),
        "breakdown_us": {"layer_step": round(t["ms_step"] * 1e3, 3),
                         "prologue": round(t["pro_ms"] * 1e3, 3),
                         "gemm": round(t["gemm_ms"] * 1e3, 3),
                         "prologue_GBps": round(t["bytes_pro"] / (t["pro_ms"] * 1e-3) / 1e9, 1),
                         "timed_region_wall_ms": round(t["ms_wall"], 3),
                         "layer_step_spread": t["spread"]},
        "roofline": t["roofline"],
        "cpu_baseline": cpu,
        "clock_power": t["clock_power"],
        "hbm_copy_reference": hbm_ref,
        "library_reference": libref,
        "ablation": ablation,
        "ffn_block": ffn,
        "fp8_variant": fp8,
        "outlier_decomposition": decomp,
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


def st_decode(w):
    return w.M <= 32


if __name__ == "__main__":
    main()
