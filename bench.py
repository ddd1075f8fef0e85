"""Benchmark: one PixArt-style DiT block's linears in NVFP4 W4A4 on one MI355X.

A step is the hot path for every linear of the block (qkv 1152->3456, proj 1152->1152,
fc1 1152->4608, fc2 4608->1152 at M = 4096 tokens): dynamic NVFP4 quantization of the bf16
activation (amax pass + quantize pass) followed by the W4A4 GEMM with bf16 output.  Weights are
quantized and prepacked once before timing (offline, as a deployed model ships them).  Inputs are
seeded synthetic tensors resident in device memory before the timed region.

The step's 12 kernel launches (amax, encode and GEMM per linear) are captured in a HIP graph,
10 steps per graph (the largest divisor of K up to 10), and the graph is replayed, so host launch
overhead is not part of the measurement and each replay's own launch latency is paid once per 10
steps, as in a graph of a whole forward pass; the same K steps with one step per graph are
reported beside the value.  Every replay is checked bit-for-bit against an eager run first.

Prints one JSON line: `value` is the block's GEMM work (sum of 2 M N K) divided by the measured
step time (quantization included).  `roofline` describes the dominant GEMM launch, whose average
duration is measured with HIP events around graph replays of back-to-back launches of that kernel
on the stream it runs on.  `cpu_baseline` times the CPU oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
T_START = time.perf_counter()
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s + quantize GB/s at DiT shapes; % of MFMA/HBM roofline"
PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense FP4 matrix peak (the block-scaled MXFP4 instruction)


def progress(msg):
    """One line per finished section on stderr (stdout carries only the JSON result)."""
    print(f"[bench] {msg} ({time.perf_counter() - T_START:.1f} s)", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kernel-reps", type=int, default=20, help="launches per per-kernel timing graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows of the CPU oracle's row samples (0: 256)")
    ap.add_argument("--no-hbm", action="store_true", help="skip the bandwidth-bound kernel section")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP4 section")
    ap.add_argument("--no-requant", action="store_true", help="skip the fused-requantization section")
    ap.add_argument("--no-blocks", action="store_true", help="skip the 32/64-value block section")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the video-DiT W4A4 and the matrix-bound W4A16 section")
    ap.add_argument("--kernel-probe", action="store_true",
                    help="only launch one GEMM call (--probe-shape) and a 256 MiB device copy, --steps times each "
                         "(the workload of the rocprofv3 counter passes)")
    ap.add_argument("--probe-shape", default="fc2", choices=sorted(PROBE_SHAPES),
                    help="the call --kernel-probe launches: a PixArt block linear (W4A4, bf16 out), the video-DiT "
                         "qkv linear (W4A4), or the weight-only up projection at M = 256 / 4096 (W4A16)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the NVFP4 hot path here is a single-device kernel set "
              "(no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_quantized_gemm_amd as nv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- setup (untimed): inputs, offline weight prep, outputs, workspaces ----------------------
    layers = []
    for name, x, w in workloads.pixart():
        M, K = x.shape
        N = w.shape[0]
        wp, ws, wS = nv.nvfp4_quantize(w.to(dev))
        bp = nv.nvfp4_prepack_weight(wp, ws)
        del wp, ws
        L = dict(name=name, M=M, N=N, K=K, x=x.to(dev), bp=bp, wS=wS,
                 packed=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                 scales=torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                 S=torch.empty(1, dtype=torch.float32, device=dev),
                 qws=torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev),
                 y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                 gws=None, w_cpu=w, x_cpu=x)
        need = nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K)
        if need:
            L["gws"] = torch.empty(need, dtype=torch.uint8, device=dev)
        layers.append(L)
    torch.cuda.synchronize()

    def quantize(L):
        nv.nvfp4_quantize(L["x"], L["S"], static=False, packed=L["packed"], scales=L["scales"],
                          workspace=L["qws"])

    def gemm(L):
        nv.nvfp4_gemm(nv.W4A4, L["packed"], L["scales"], L["S"], L["bp"], L["wS"], L["N"], L["K"],
                      torch.bfloat16, out=L["y"], workspace=L["gws"])

    def step():
        for L in layers:
            quantize(L)
            gemm(L)

    if args.kernel_probe:
        for L in layers:
            quantize(L)
        kernel_probe(args, layers, gemm)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager = [L["y"].clone() for L in layers]

    # ---- capture G steps per graph (G the largest divisor of K up to 10: each replay's launch
    # latency is paid once per G steps, as in a graph of a whole forward pass); check replays
    # against the eager result -----------------------------------------------------------------------
    G = max(d for d in range(1, min(10, args.steps) + 1) if args.steps % d == 0)
    side = torch.cuda.Stream()

    def capture(nsteps):
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(nsteps):
                    step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for _ in range(3):
            for L in layers:
                L["y"].zero_()
            g.replay()
            torch.cuda.synchronize()
            for L, ref in zip(layers, eager):
                if not torch.equal(L["y"], ref):
                    raise RuntimeError(f"graph replay differs from eager result for {L['name']}")
        return g

    graph = capture(G)
    graph1 = capture(1) if G > 1 else graph

    # ---- timed region: K steps = K / G replays ------------------------------------------------------
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps // G):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    # the same K steps with one step per graph (reported beside the value, not used for it)
    t0.record(stream)
    for _ in range(args.steps):
        graph1.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step_1 = t0.elapsed_time(t1) / args.steps

    # ---- the same step with calibrated (static) activation scales: each S taken from the dynamic
    # run, so one encode pass per quantize instead of amax + encode; the outputs must not change ---
    for L in layers:
        L["S_cal"] = L["S"].clone()

    def step_static():
        for L in layers:
            nv.nvfp4_quantize(L["x"], L["S_cal"], static=True, packed=L["packed"], scales=L["scales"])
            nv.nvfp4_gemm(nv.W4A4, L["packed"], L["scales"], L["S_cal"], L["bp"], L["wS"], L["N"], L["K"],
                          torch.bfloat16, out=L["y"], workspace=L["gws"])

    side.wait_stream(torch.cuda.current_stream())
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(gs, stream=side):
            for _ in range(G):
                step_static()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for L in layers:
        L["y"].zero_()
    gs.replay()
    torch.cuda.synchronize()
    for L, ref in zip(layers, eager):
        if not torch.equal(L["y"], ref):
            raise RuntimeError(f"static-scale step differs from the dynamic result for {L['name']}")
    t0.record(stream)
    for _ in range(args.steps // G):
        gs.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step_static = t0.elapsed_time(t1) / args.steps
    del gs

    # ---- per-kernel durations: graphs of back-to-back launches of one kernel -----------------------
    def kernel_us(fn, L):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(args.kernel_reps):
                    fn(L)
        torch.cuda.synchronize()
        g.replay()  # warm
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * args.kernel_reps)

    flops_step = sum(2.0 * L["M"] * L["N"] * L["K"] for L in layers)
    breakdown = {}
    for L in layers:
        q_us = kernel_us(quantize, L)
        g_us = kernel_us(gemm, L)
        qbytes = L["M"] * L["K"] * (2 + 2 + 0.5625)  # amax read + quantize read + codes/scales write
        flops = 2.0 * L["M"] * L["N"] * L["K"]
        breakdown[L["name"]] = dict(
            M=L["M"], N=L["N"], K=L["K"],
            quantize_us=round(q_us, 2), quantize_GBps=round(qbytes / (q_us * 1e-6) / 1e9, 1),
            gemm_us=round(g_us, 2), gemm_TFLOPs=round(flops / (g_us * 1e-6) / 1e12, 1),
            gemm_frac=round(flops / (g_us * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4))
    d = breakdown[DOMINANT]
    traffic = measured_traffic()
    roofline = dict(bound="mfma", achieved=d["gemm_TFLOPs"], peak=PEAK_FP16_TFLOPS, unit="TFLOP/s",
                    frac=round(d["gemm_TFLOPs"] / PEAK_FP16_TFLOPS, 4),
                    traffic=None if traffic is None else int(traffic),
                    kernel=f"nvfp4_gemm W4A4 {DOMINANT} M={d['M']} N={d['N']} K={d['K']} bf16 out "
                           f"(launches: {gemm_kernels(nv, d)})",
                    avg_launch_us=d["gemm_us"], algorithmic_flops_per_launch=2 * d["M"] * d["N"] * d["K"],
                    algorithmic_bytes_per_launch=int(d["M"] * d["K"] * 0.5625 + d["N"] * d["K"] * 0.5625
                                                     + d["M"] * d["N"] * 2),
                    kernel_source_sha256=kernel_source_hash())
    q_total_bytes = sum(L["M"] * L["K"] * 4.5625 for L in layers)
    q_total_us = sum(v["quantize_us"] for v in breakdown.values())
    g_total_us = sum(v["gemm_us"] for v in breakdown.values())

    out = {
        "metric": METRIC,
        "value": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "PixArt-style DiT block linears, W4A4, bf16 in/out", "M": 4096, "hidden": 1152,
                   "linears": {L["name"]: [L["K"], L["N"]] for L in layers}, "parallelism": "none (1 GPU)",
                   "timing": f"HIP-graph replay, {G} steps per graph"},
        "ms_per_step_one_step_per_graph": round(ms_step_1, 4),
        "static_activation_scales": {
            "ms_per_step": round(ms_step_static, 4),
            "TFLOPs": round(flops_step / (ms_step_static * 1e-3) / 1e12, 2),
            "note": "the same step with each activation's S calibrated (taken from the dynamic run): one "
                    "encode pass per quantize; outputs identical to the dynamic step"},
        "roofline": roofline,
        "quantize": {"achieved_GBps": round(q_total_bytes / (q_total_us * 1e-6) / 1e9, 1), "peak_GBps": PEAK_HBM_GBS,
                     "frac": round(q_total_bytes / (q_total_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "bytes_per_elem": 4.5625, "note": "dynamic: amax pass + quantize pass"},
        "gemm_TFLOPs_all_linears": round(flops_step / (g_total_us * 1e-6) / 1e12, 1),
        "breakdown": breakdown,
        "wall_s_timed": round(wall, 4),
    }
    progress("block step timed")
    if not args.no_hbm:
        out["hbm_kernels"] = hbm_kernels(side, stream)
        progress("bandwidth section done")
    if not args.no_mx:
        out["mxfp4"] = mxfp4_section(layers, side, stream, args.kernel_reps)
        progress("MXFP4 section done")
    if not args.no_requant:
        out["fused_requant"] = requant_section(layers, side, stream, args.kernel_reps)
        progress("fused-requantization section done")
    if not args.no_blocks:
        out["block_sizes"] = block_size_section(layers, side, stream, args.kernel_reps)
        progress("block-size section done")
    if not args.no_other:
        out["other_configs"] = other_configs_section(side, stream, args.kernel_reps)
        progress("video-DiT / weight-only section done")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, args.cpu_rows)
        progress("CPU oracle baseline done")
    print(json.dumps(out), flush=True)


DOMINANT = "fc2"  # the block's longest GEMM call (4608 -> 1152)
# --kernel-probe shapes: (mode, M, N, K); the PixArt linears use the block's own inputs
PROBE_SHAPES = {"qkv": None, "proj": None, "fc1": None, "fc2": None,
                "video_qkv": ("W4A4", 10240, 9216, 3072), "w4a16_up_256": ("W4A16", 256, 12288, 3072),
                "w4a16_up_4096": ("W4A16", 4096, 12288, 3072),
                "mx_qkv": ("MX", "qkv"), "mx_fc2": ("MX", "fc2"), "mx_cube": ("MX", 8192, 8192, 8192)}
COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4a4_fc2_traffic.json")
KERNEL_SOURCES = ("gemm.hip", "launch.hpp", "common.hpp", "epilogue.hpp", "quant_core.hpp")  # the dominant GEMM call's code


def gemm_kernels(nv, d):
    """The kernels one call launches at this shape (a split-K plan needs a workspace)."""
    ws = nv.nvfp4_gemm_workspace_bytes(nv.W4A4, d["M"], d["N"], d["K"])
    if ws:
        return f"k_gemm_tiled split-K x{ws // (4 * d['M'] * d['N'])} + k_splitk_reduce"
    return "k_gemm_tiled, one launch"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "nvfp4_quantized_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per call of the dominant GEMM from the committed counter passes, scaled by the
    counters' reading for a plain copy of known size; None if the kernel changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        t = json.load(fh)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t["fetch_bytes_per_call"] / t["copy_fetch_factor"] + t["write_bytes_per_call"] / t["copy_write_factor"]


def kernel_probe(args, layers, gemm):
    """Counter-pass workload: one GEMM call (--probe-shape), then a plain device copy of COPY_BYTES."""
    import torch

    import nvfp4_quantized_gemm_amd as nv
    import workloads

    name = args.probe_shape
    if PROBE_SHAPES[name] is None:
        L = next(L for L in layers if L["name"] == name)
        print(f"probe: nvfp4_gemm W4A4 {name} M={L['M']} N={L['N']} K={L['K']} x {args.steps}", flush=True)
        call = lambda: gemm(L)
    elif PROBE_SHAPES[name][0] == "MX":
        # MXFP4 GEMM: a PixArt linear on the block's own inputs, or a random cube
        if len(PROBE_SHAPES[name]) == 2:
            L = next(L for L in layers if L["name"] == PROBE_SHAPES[name][1])
            xa, wb = L["x"], L["w_cpu"].cuda()
        else:
            _, M, N, K = PROBE_SHAPES[name]
            g = torch.Generator().manual_seed(5)
            xa = torch.randn(M, K, generator=g).to(torch.bfloat16).cuda()
            wb = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16).cuda()
        a, a_s = nv.nvfp4_mx_quantize(xa)
        b, b_s = nv.nvfp4_mx_quantize(wb)
        y = torch.empty((xa.shape[0], wb.shape[0]), dtype=torch.bfloat16, device="cuda")
        print(f"probe: nvfp4_mx_gemm {name} M={xa.shape[0]} N={wb.shape[0]} K={xa.shape[1]} x {args.steps}",
              flush=True)
        call = lambda: nv.nvfp4_mx_gemm(a, a_s, b, b_s, out=y)
    else:
        mode, M, N, K = PROBE_SHAPES[name]
        g = torch.Generator().manual_seed(5)
        w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16).cuda()
        wp, ws, wS = nv.nvfp4_quantize(w)
        bp = nv.nvfp4_prepack_weight(wp, ws)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        if mode == "W4A4":
            x = workloads.video_activation(M, K, g).cuda()
            pa, sa, Sa = nv.nvfp4_quantize(x)
            ws_ = torch.empty(max(1, nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K)), dtype=torch.uint8,
                              device="cuda")
            call = lambda: nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, torch.bfloat16, out=y, workspace=ws_)
        else:
            a = torch.randn(M, K, generator=g).to(torch.bfloat16).cuda()
            ws_ = torch.empty(max(1, nv.nvfp4_gemm_workspace_bytes(nv.W4A16, M, N, K)), dtype=torch.uint8,
                              device="cuda")
            call = lambda: nv.nvfp4_gemm(nv.W4A16, a, None, None, bp, wS, N, K, torch.bfloat16, out=y, workspace=ws_)
        print(f"probe: nvfp4_gemm {mode} {name} M={M} N={N} K={K} x {args.steps}", flush=True)
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    print(f"probe: device copy of {COPY_BYTES} bytes x {args.steps}", flush=True)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("probe: done", flush=True)


def time_graph(fns, side, stream, replays=5):
    """Average duration of one call when the calls in `fns` are captured back to back in one graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for fn in fns:
                fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (replays * len(fns))


def hbm_kernels(side, stream):
    """Bandwidth-bound calls at sizes well beyond the 256 MB last-level cache: quantize (dynamic and
    static), dequantize and fake quantization (QAT) of a 32768 x 12288 bf16 tensor, and the
    weight-only GEMM with M = 1 and 16 rows cycling through 32 copies of the prepacked weight
    (~680 MB)."""
    import torch

    import nvfp4_quantized_gemm_amd as nv
    import workloads

    dev = "cuda"
    res = {}

    def entry(us, nbytes):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us": round(us, 2), "GBps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                "bytes": int(nbytes)}

    M, K = 32768, 12288
    x = workloads.sweep(M, K).to(dev)
    packed = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    S = torch.empty(1, dtype=torch.float32, device=dev)
    Sst = torch.full((1,), workloads.SWEEP_STATIC_S, dtype=torch.float32, device=dev)
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    n = M * K
    reps = 10
    us = time_graph([lambda: nv.nvfp4_quantize(x, S, static=False, packed=packed, scales=scales, workspace=qws)] * reps,
                    side, stream)
    res[f"quantize_dynamic_bf16_{M}x{K}"] = entry(us, n * (2 + 2 + 0.5625))
    us = time_graph([lambda: nv.nvfp4_quantize(x, Sst, static=True, packed=packed, scales=scales)] * reps, side, stream)
    res[f"quantize_static_bf16_{M}x{K}"] = entry(us, n * (2 + 0.5625))
    us = time_graph([lambda: nv.nvfp4_dequantize(packed, scales, Sst, torch.bfloat16, out=y)] * reps, side, stream)
    res[f"dequantize_bf16_{M}x{K}"] = entry(us, n * (0.5625 + 2))
    yq = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    us = time_graph([lambda: nv.nvfp4_fake_quantize(x, Sst, static=True, out=yq)] * reps, side, stream)
    res[f"fake_quantize_static_bf16_{M}x{K}"] = entry(us, n * (2 + 2))
    us = time_graph([lambda: nv.nvfp4_fake_quantize(x, S, static=False, out=yq, workspace=qws)] * reps, side, stream)
    res[f"fake_quantize_dynamic_bf16_{M}x{K}"] = entry(us, n * (2 + 2 + 2))
    del yq
    # The sweep's planted 10.5 makes the dynamic S exactly 2^-8, which keeps every decision on the
    # cheap exact-tie path.  A plain N(0, 1) tensor of the same size gives a generic S.
    g = torch.Generator().manual_seed(41)
    x.copy_(torch.randn(M, K, generator=g).to(torch.bfloat16))
    us = time_graph([lambda: nv.nvfp4_quantize(x, S, static=False, packed=packed, scales=scales, workspace=qws)] * reps,
                    side, stream)
    res[f"quantize_dynamic_bf16_{M}x{K}_generic_S"] = entry(us, n * (2 + 2 + 0.5625))
    res[f"quantize_dynamic_bf16_{M}x{K}_generic_S"]["S"] = float(S.item())
    us = time_graph([lambda: nv.nvfp4_quantize(x, S, static=True, packed=packed, scales=scales)] * reps, side, stream)
    res[f"quantize_static_bf16_{M}x{K}_generic_S"] = entry(us, n * (2 + 0.5625))
    # measured floors beside 8 TB/s: a device copy of the same bf16 tensor (read + write)
    us = time_graph([lambda: y.copy_(x)] * reps, side, stream)
    copy_big = entry(us, n * 4)
    res[f"copy_bf16_{M}x{K}"] = copy_big
    del x, packed, scales, y
    torch.cuda.empty_cache()

    copies = 32
    # the weight-only calls' floor: a copy of one weight's 21 MB as a dependent launch, rotating over
    # 32 source buffers like the GEMM calls below
    wb = 21 << 20
    srcs = [torch.empty(wb, dtype=torch.uint8, device=dev) for _ in range(copies)]
    dst = torch.empty(wb, dtype=torch.uint8, device=dev)
    us = time_graph([(lambda s_=s_: dst.copy_(s_)) for s_ in srcs], side, stream)
    copy_small = entry(us, 2 * wb)
    res["copy_21MiB_dependent_launch"] = copy_small
    del srcs, dst
    for name, (w, acts) in workloads.w4a16(ms=(1, 16)).items():
        N, Kw = w.shape
        wp, ws, wS = nv.nvfp4_quantize(w.to(dev))
        bp = nv.nvfp4_prepack_weight(wp, ws)
        bps = [bp.clone() for _ in range(copies)]
        del wp, ws, bp
        for m, a in acts.items():
            ad = a.to(dev)
            out = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            need = nv.nvfp4_gemm_workspace_bytes(nv.W4A16, m, N, Kw)
            gws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            fns = [(lambda b=b: nv.nvfp4_gemm(nv.W4A16, ad, None, None, b, wS, N, Kw, torch.bfloat16, out=out,
                                              workspace=gws)) for b in bps]
            us = time_graph(fns, side, stream)
            e = entry(us, 0.5625 * N * Kw + 2 * m * Kw + 2 * m * N)
            e["TFLOPs"] = round(2.0 * m * N * Kw / (us * 1e-6) / 1e12, 2)
            e["time_vs_copy_21MiB"] = round(us / copy_small["us"], 3)  # < 1: faster than the copy
            res[f"w4a16_{name}_M{m}_N{N}_K{Kw}"] = e
        del bps
        torch.cuda.empty_cache()
    # the bandwidth calls of the big tensor against the measured copy rate
    for k, v in res.items():
        if k.endswith(f"{M}x{K}") or k.endswith("_generic_S"):
            v["frac_of_copy"] = round(v["GBps"] / copy_big["GBps"], 4)
    return res


def mxfp4_section(layers, side, stream, reps):
    """The same block in MXFP4 (32-value E8M0 blocks, block-scaled FP4 matrix instruction): per
    linear, the activation quantize and the GEMM (weights quantized beforehand), each timed as
    back-to-back launches in one graph; the step is their sum."""
    import torch

    import nvfp4_quantized_gemm_amd as nv

    res = {}
    step_us = 0.0
    flops_step = 0.0
    for L in layers:
        M, N, K = L["M"], L["N"], L["K"]
        b, bs = nv.nvfp4_mx_quantize(L["w_cpu"].to(L["x"].device))
        a = torch.empty((M, K // 2), dtype=torch.uint8, device=L["x"].device)
        asc = torch.empty((M, K // 32), dtype=torch.uint8, device=L["x"].device)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=L["x"].device)
        q_us = time_graph([lambda: nv.nvfp4_mx_quantize(L["x"], packed=a, scales=asc)] * reps, side, stream)
        g_us = time_graph([lambda: nv.nvfp4_mx_gemm(a, asc, b, bs, out=y)] * reps, side, stream)
        flops = 2.0 * M * N * K
        tf = flops / (g_us * 1e-6) / 1e12
        res[L["name"]] = {"quantize_us": round(q_us, 2), "gemm_us": round(g_us, 2), "gemm_TFLOPs": round(tf, 1),
                          "gemm_frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4)}
        step_us += q_us + g_us
        flops_step += flops
    res["block_step_us"] = round(step_us, 2)
    res["block_TFLOPs"] = round(flops_step / (step_us * 1e-6) / 1e12, 1)
    res["peak_TFLOPs"] = PEAK_FP4_TFLOPS
    return res


def requant_section(layers, side, stream, reps):
    """The block's MLP pair (fc1 -> fc2) with the fc1 GEMM writing NVFP4 directly (tanh GELU, static
    output scale calibrated on an eager run) against the unfused sequence the step uses (fc1 with
    bf16 output, dynamic quantize of that output, fc2).  The unfused sequence does no GELU, so the
    fused one does strictly more work.  Each piece is timed as back-to-back launches in one graph."""
    import torch

    import nvfp4_quantized_gemm_amd as nv

    by = {L["name"]: L for L in layers}
    f1, f2 = by["fc1"], by["fc2"]
    dev = f1["x"].device
    M, N1, K1 = f1["M"], f1["N"], f1["K"]
    # fc1 activation (quantized as in the step) and the bf16 fc1 output of the unfused path
    nv.nvfp4_quantize(f1["x"], f1["S"], static=False, packed=f1["packed"], scales=f1["scales"], workspace=f1["qws"])
    h16 = torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
    hp = torch.empty((M, N1 // 2), dtype=torch.uint8, device=dev)
    hs = torch.empty((M, N1 // 16), dtype=torch.uint8, device=dev)
    hS = torch.empty(1, dtype=torch.float32, device=dev)
    hws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, N1), dtype=torch.uint8, device=dev)
    y2 = torch.empty((M, f2["N"]), dtype=torch.bfloat16, device=dev)
    # calibration: the static scale of the GELU output, from one eager fp32 pass
    hy = torch.empty((M, N1), dtype=torch.float32, device=dev)
    cal = torch.ones(1, dtype=torch.float32, device=dev)
    nv.nvfp4_gemm_requant(nv.W4A4, f1["packed"], f1["scales"], f1["S"], f1["bp"], f1["wS"], N1, K1, cal,
                          act=nv.ACT_GELU_TANH, packed=hp, scales=hs, y=hy)
    So = (hy.abs().max() / 2688.0).reshape(1).contiguous()
    del hy
    rws = nv.nvfp4_gemm_requant_workspace_bytes(nv.W4A4, M, N1, K1)
    rws_t = torch.empty(max(rws, 1), dtype=torch.uint8, device=dev)

    def fc1_bf16():
        nv.nvfp4_gemm(nv.W4A4, f1["packed"], f1["scales"], f1["S"], f1["bp"], f1["wS"], N1, K1, torch.bfloat16,
                      out=h16, workspace=f1["gws"])

    def quant_dyn():
        nv.nvfp4_quantize(h16, hS, static=False, packed=hp, scales=hs, workspace=hws)

    def fc1_requant():
        nv.nvfp4_gemm_requant(nv.W4A4, f1["packed"], f1["scales"], f1["S"], f1["bp"], f1["wS"], N1, K1, So,
                              act=nv.ACT_GELU_TANH, packed=hp, scales=hs, workspace=rws_t)

    def fc2_from_h(S):
        nv.nvfp4_gemm(nv.W4A4, hp, hs, S, f2["bp"], f2["wS"], f2["N"], f2["K"], torch.bfloat16, out=y2,
                      workspace=f2["gws"])

    res = {"M": M, "fc1": [N1, K1], "fc2": [f2["N"], f2["K"]], "static_S": float(So.item())}
    res["fc1_gemm_bf16_us"] = round(time_graph([fc1_bf16] * reps, side, stream), 2)
    res["fc2_act_quantize_dynamic_us"] = round(time_graph([quant_dyn] * reps, side, stream), 2)
    res["fc1_gemm_gelu_requant_us"] = round(time_graph([fc1_requant] * reps, side, stream), 2)
    res["mlp_unfused_us"] = round(time_graph([fc1_bf16, quant_dyn, lambda: fc2_from_h(hS)] * 4, side, stream) * 3, 2)
    res["mlp_fused_us"] = round(time_graph([fc1_requant, lambda: fc2_from_h(So)] * 4, side, stream) * 2, 2)
    return res


def block_size_section(layers, side, stream, reps):
    """The step with 32 and 64 values per E4M3 scale byte (activations and weights alike): per linear,
    the dynamic activation quantize and the W4A4 GEMM, each timed as back-to-back launches in one
    graph; the step is their sum.  Also the dynamic quantize of a 32768 x 12288 bf16 N(0, 1) tensor
    (generic S) at each block size, against HBM."""
    import torch

    import nvfp4_quantized_gemm_amd as nv

    res = {}
    for b in (32, 64):
        r = {}
        step_us = 0.0
        flops_step = 0.0
        for L in layers:
            M, N, K = L["M"], L["N"], L["K"]
            dev = L["x"].device
            wp, ws, wS = nv.nvfp4_quantize(L["w_cpu"].to(dev), block_size=b)
            bp = nv.nvfp4_prepack_weight(wp, ws)
            del wp, ws
            pa = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            sa = torch.empty((M, K // b), dtype=torch.uint8, device=dev)
            Sa = torch.empty(1, dtype=torch.float32, device=dev)
            q_us = time_graph([lambda: nv.nvfp4_quantize(L["x"], Sa, static=False, packed=pa, scales=sa,
                                                         workspace=L["qws"], block_size=b)] * reps, side, stream)
            g_us = time_graph([lambda: nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, torch.bfloat16,
                                                     out=L["y"], workspace=L["gws"])] * reps, side, stream)
            flops = 2.0 * M * N * K
            r[L["name"]] = {"quantize_us": round(q_us, 2), "gemm_us": round(g_us, 2),
                            "gemm_TFLOPs": round(flops / (g_us * 1e-6) / 1e12, 1)}
            step_us += q_us + g_us
            flops_step += flops
        r["block_step_us"] = round(step_us, 2)
        r["block_TFLOPs"] = round(flops_step / (step_us * 1e-6) / 1e12, 1)
        res[f"b{b}"] = r
    torch.cuda.empty_cache()

    M, K = 32768, 12288
    dev = layers[0]["x"].device
    g = torch.Generator().manual_seed(41)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev)
    packed = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    S = torch.empty(1, dtype=torch.float32, device=dev)
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    for b in (16, 32, 64):
        scales = torch.empty((M, K // b), dtype=torch.uint8, device=dev)
        us = time_graph([lambda: nv.nvfp4_quantize(x, S, static=False, packed=packed, scales=scales, workspace=qws,
                                                   block_size=b)] * 10, side, stream)
        nbytes = M * K * (2 + 2 + 0.5 + 1.0 / b)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"quantize_dynamic_bf16_{M}x{K}_generic_S_b{b}"] = {
            "us": round(us, 2), "GBps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": int(nbytes)}
        del scales
    del x, packed, qws
    torch.cuda.empty_cache()
    return res


def other_configs_section(side, stream, reps):
    """The tiny linear (M = 256, K = N = 1152, fp32 activation and output); the video-DiT linears (M = 10240 tokens, hidden 3072; Student-t activations with log-normal
    channel scales, seed 3) as in the step: dynamic activation quantize + W4A4 GEMM with bf16 output
    per linear; and the weight-only GEMM at the matrix-bound row counts M = 256 and 4096 (seed 2
    weights).  Each call is timed as back-to-back launches in one graph, the better of two timings."""
    import torch

    import nvfp4_quantized_gemm_amd as nv
    import workloads

    dev = "cuda"
    res = {"tiny_w4a4": {}, "video_dit_w4a4": {}, "w4a16_matrix_bound": {}}
    # the tiny linear (X fp32 [256, 1152], W [1152, 1152], seed 0): dynamic quantize of X, W4A4 GEMM
    # with fp32 output
    x, w = workloads.tiny()
    M, K = x.shape
    N = w.shape[0]
    xd = x.to(dev)
    wp, ws, wS = nv.nvfp4_quantize(w.to(dev))
    bp = nv.nvfp4_prepack_weight(wp, ws)
    pa = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    Sa = torch.empty(1, dtype=torch.float32, device=dev)
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    gws = torch.empty(max(1, nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K)), dtype=torch.uint8, device=dev)
    q_us = min(time_graph([lambda: nv.nvfp4_quantize(xd, Sa, static=False, packed=pa, scales=sa, workspace=qws)]
                          * reps, side, stream) for _ in range(2))
    g_us = min(time_graph([lambda: nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, torch.float32, out=y,
                                                 workspace=gws)] * reps, side, stream) for _ in range(2))
    tf = 2.0 * M * N * K / (g_us * 1e-6) / 1e12
    res["tiny_w4a4"] = {"M": M, "N": N, "K": K, "quantize_us": round(q_us, 2), "gemm_us": round(g_us, 2),
                        "gemm_TFLOPs": round(tf, 1), "gemm_frac": round(tf / PEAK_FP16_TFLOPS, 4)}
    del xd, wp, ws, bp, pa, sa, y, gws, qws
    step_us, flops_step = 0.0, 0.0
    for name, x, w in workloads.video():
        M, K = x.shape
        N = w.shape[0]
        xd = x.to(dev)
        wp, ws, wS = nv.nvfp4_quantize(w.to(dev))
        bp = nv.nvfp4_prepack_weight(wp, ws)
        del wp, ws
        pa = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        sa = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
        Sa = torch.empty(1, dtype=torch.float32, device=dev)
        qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gws = torch.empty(max(1, nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K)), dtype=torch.uint8, device=dev)
        # the first graph of a shape runs while the clocks settle: keep the second of two timings
        q_us = min(time_graph([lambda: nv.nvfp4_quantize(xd, Sa, static=False, packed=pa, scales=sa,
                                                         workspace=qws)] * reps, side, stream) for _ in range(2))
        g_us = min(time_graph([lambda: nv.nvfp4_gemm(nv.W4A4, pa, sa, Sa, bp, wS, N, K, torch.bfloat16, out=y,
                                                     workspace=gws)] * reps, side, stream) for _ in range(2))
        flops = 2.0 * M * N * K
        tf = flops / (g_us * 1e-6) / 1e12
        res["video_dit_w4a4"][name] = {"M": M, "N": N, "K": K, "quantize_us": round(q_us, 2),
                                       "gemm_us": round(g_us, 2), "gemm_TFLOPs": round(tf, 1),
                                       "gemm_frac": round(tf / PEAK_FP16_TFLOPS, 4)}
        step_us += q_us + g_us
        flops_step += flops
        del xd, bp, pa, sa, y, gws, qws
        torch.cuda.empty_cache()
    res["video_dit_w4a4"]["linears_TFLOPs"] = round(flops_step / (step_us * 1e-6) / 1e12, 1)
    for name, (w, acts) in workloads.w4a16(ms=(256, 4096)).items():
        N, K = w.shape
        wp, ws, wS = nv.nvfp4_quantize(w.to(dev))
        bp = nv.nvfp4_prepack_weight(wp, ws)
        del wp, ws
        for m, a in acts.items():
            ad = a.to(dev)
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            gws = torch.empty(max(1, nv.nvfp4_gemm_workspace_bytes(nv.W4A16, m, N, K)), dtype=torch.uint8,
                              device=dev)
            us = min(time_graph([lambda: nv.nvfp4_gemm(nv.W4A16, ad, None, None, bp, wS, N, K, torch.bfloat16,
                                                       out=y, workspace=gws)] * reps, side, stream) for _ in range(2))
            tf = 2.0 * m * N * K / (us * 1e-6) / 1e12
            res["w4a16_matrix_bound"][f"{name}_M{m}_N{N}_K{K}"] = {"us": round(us, 2), "TFLOPs": round(tf, 1),
                                                                  "frac": round(tf / PEAK_FP16_TFLOPS, 4)}
        del bp
        torch.cuda.empty_cache()
    return res


def host_identity():
    """CPU model name, logical CPUs of the host, and the CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(layers, rows):
    """The CPU oracle (plain C, OpenMP over rows, fp64-accumulated GEMM) on this machine's host cores,
    timed with all the threads this job may use and with one thread.  The headline value is the
    whole PixArt block on all threads (every row of every linear: the activation's tensor scale,
    quantize, dequantize and the GEMM against the offline-quantized weight).  Alongside: the tiny
    fp32 linear end to end, single-thread rates on a leading-row sample (extrapolated linearly, and
    labelled so), the video-DiT linears and the weight-only GEMM on leading-row samples, and the
    quantize / dequantize rate on a sweep tensor.  `rows` caps the sampled rows (0: 256)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    host = host_identity()
    threads = max(1, min(host["usable_cpus"], int(os.environ.get("OMP_NUM_THREADS", host["usable_cpus"]))))
    srows = rows if rows > 0 else 256
    bf16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)

    def linear(x, B, nthreads, nrows=None):
        """tensor scale over all of x, then quantize + dequantize + GEMM for the first nrows rows"""
        S = oracle.tensor_scale(x)
        xs = x if nrows is None else np.ascontiguousarray(x[:nrows])
        p, sc, _ = oracle.quantize(xs, S=S, threads=nthreads)
        A, _ = oracle.dequantize(p, sc, S, threads=nthreads)
        oracle.gemm(A, B, threads=nthreads)
        return 2.0 * xs.shape[0] * B.shape[0] * B.shape[1]

    def weight(w, nthreads):
        bp, bs, bS = oracle.quantize(w, threads=nthreads)
        return oracle.dequantize(bp, bs, bS, threads=nthreads)[0]

    res = {"kind": "oracle", "host": host, "threads": threads}
    # PixArt block (the benchmark's workload): full on all threads; one thread on a row sample
    prep = [(bf16(L["x_cpu"]), weight(bf16(L["w_cpu"]), threads)) for L in layers]
    t = time.perf_counter()
    flops = sum(linear(x, B, threads) for x, B in prep)
    dt = time.perf_counter() - t
    value = flops / dt / 1e12
    t = time.perf_counter()
    f1 = sum(linear(x, B, 1, srows) for x, B in prep)
    dt1 = time.perf_counter() - t
    res["pixart_block"] = {"all_threads_s": round(dt, 3), "all_threads_TFLOPs": round(value, 6),
                           "one_thread_TFLOPs": round(f1 / dt1 / 1e12, 6),
                           "one_thread_s_extrapolated": round(dt1 * layers[0]["M"] / srows, 2),
                           "one_thread_sample": f"first {srows} of {layers[0]['M']} rows of every linear, "
                                                f"{dt1:.2f} s, extrapolated linearly"}
    # tiny fp32 linear end to end (weight quantization included): the seconds-scale oracle run
    x, w = workloads.tiny()
    for n, key in ((threads, "all_threads_s"), (1, "one_thread_s")):
        t = time.perf_counter()
        linear(x.numpy(), weight(w.numpy(), n), n)
        res.setdefault("tiny_w4a4", {})[key] = round(time.perf_counter() - t, 4)
    # video-DiT linears and the weight-only GEMM: leading-row samples on all threads, extrapolated
    g = torch.Generator().manual_seed(3)
    vid, vflops, vt = {}, 0.0, 0.0
    for name, N, K in workloads.VIDEO_LINEARS:
        xv = bf16(workloads.video_activation(srows, K, g))
        B = weight(bf16((0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)), threads)
        t = time.perf_counter()
        f = linear(xv, B, threads)
        vt += time.perf_counter() - t
        vflops += f
    res["video_dit"] = {"all_threads_TFLOPs": round(vflops / vt / 1e12, 6),
                        "all_threads_s_extrapolated": round(vt * workloads.VIDEO_M / srows, 2),
                        "sample": f"{srows} rows of each linear (same distribution as the 10240-row activations), "
                                  f"{vt:.2f} s, extrapolated linearly"}
    w16 = {}
    for name, (w, acts) in workloads.w4a16(ms=(1, 16, srows)).items():
        B = weight(w.numpy(), threads)
        for m, a in acts.items():
            A = oracle.bf16_to_f32(bf16(a))
            t = time.perf_counter()
            oracle.gemm(A, B, threads=threads)
            dtm = time.perf_counter() - t
            w16[f"{name}_M{m}"] = {"s": round(dtm, 4), "TFLOPs": round(2.0 * m * B.shape[0] * B.shape[1] / dtm / 1e12, 6)}
        w16[f"{name}_M4096_s_extrapolated"] = round(w16[f"{name}_M{srows}"]["s"] * 4096 / srows, 2)
    res["w4a16"] = w16
    # quantize + dequantize of a sweep tensor (bf16 4096 x 12288)
    xs = bf16(workloads.sweep(4096, 12288))
    t = time.perf_counter()
    p, sc, S = oracle.quantize(xs, threads=threads)
    tq = time.perf_counter() - t
    t = time.perf_counter()
    oracle.dequantize(p, sc, S, threads=threads)
    td = time.perf_counter() - t
    n = xs.size
    res["sweep_4096x12288"] = {"quantize_dynamic_GBps": round(n * 4.5625 / tq / 1e9, 2),
                               "dequantize_GBps": round(n * 2.5625 / td / 1e9, 2)}
    res["value"] = round(value, 6)
    res["unit"] = "TFLOP/s"
    res["cores"] = threads
    res["sample"] = (f"the whole PixArt block (all {layers[0]['M']} rows of every linear: tensor scale, quantize, "
                     f"dequantize, fp64-accumulated GEMM), {dt:.2f} s on {threads} threads of {host['model']}")
    return res


if __name__ == "__main__":
    main()
