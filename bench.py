"""Benchmark of the fused MoE routed-expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--tokens T]
                    [--flush-mb MB] [--no-cpu-baseline]

A step is one moe_forward call (dispatch quantisation, routing metadata, L1
GEMM + SwiGLU + L2-input quantisation, L2 GEMM, weighted combine) over one
batch of synthetic input already resident in HBM.  W untimed warm-up steps,
then exactly K steps between two synchronisations; one JSON line on stdout.

Default: every format's seeded workload in one run, one JSON line.  Its
headline is the largest single-GPU layer, DeepSeek-V3-shaped MXFP8 (8192
tokens, hidden 7168, intermediate 2048, 256 routed experts + 1 shared,
top-8); ``workloads`` holds one record of the same form per other workload:
Mixtral-8x7B-shaped BF16 (4096 tokens), the NVFP4 layer under Zipf routing
(16384 tokens), and the decode-shaped MXFP4 (W4A8) layer at 1, 8, 32, 128
and 256 tokens, each decode step timed after a 1 GiB read that evicts the
256 MB MALL.  --config runs one workload alone.

Roofline: the dominant kernel (the L1 grouped GEMM) is timed live with HIP
events recorded by the library on the stream it launches on
(moe_forward_profiled).  Its algorithmic work is 4 * S * H * I FLOPs (S real
slots; padding rows are overhead) or the weight bytes it must stream,
against MI355X's published peaks (dense MFMA BF16/FP16 2500 TFLOP/s, FP8
5000, FP4 10100; HBM 8000 GB/s).  NVFP4 runs its products on the FP16 MFMA
(exactly dequantised operands), so its fraction is of the FP16 peak, with
the FP4 peak's fraction alongside.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 5000.0, "nvfp4": 2500.0}
PEAK_FP4_TFLOPS = 10100.0
PEAK_HBM_GBS = 8000.0
HEADLINE = ("dsv3_mxfp8", None, 0)
# (workload, tokens, MB read between steps)
SUB_WORKLOADS = [("mixtral_bf16", None, 0), ("nvfp4_zipf", None, 0)] + \
    [("decode_mxfp4", t, 1024) for t in (1, 8, 32, 128, 256)]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default=None, help="one workload alone (default: every workload)")
    p.add_argument("--tokens", type=int, default=None, help="token count (decode workload)")
    p.add_argument("--flush-mb", type=int, default=0,
                   help="read this many MB between steps (evicts the weights from the 256 MB MALL without "
                        "leaving dirty lines to write back during the step)")
    p.add_argument("--block-m", type=int, default=0, help="BLOCK_M (0: the library's rule)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    p.add_argument("--cpu-tokens", type=int, default=None, help="oracle sample size (tokens)")
    p.add_argument("--route", action="store_true",
                   help="time the router top-k (moe_route) on the workload's routing shape instead")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="only run a plain device copy of this many MB (HBM counter calibration)")
    return p.parse_args()


def copy_calibration(mb, reps=3):
    """A plain device-to-device copy of known size: FETCH_SIZE / WRITE_SIZE of
    this kernel calibrate the HBM byte counters (reads mb MB, writes mb MB)."""
    src = torch.ones(mb * (1 << 20), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mb": mb, "reps": reps, "bytes_read_per_copy": mb * (1 << 20),
                      "bytes_written_per_copy": mb * (1 << 20)}), flush=True)
    return 0


KERNEL_SOURCES = ("expert_gemms_amd/csrc/gemm.hip", "expert_gemms_amd/csrc/common.h", "expert_gemms_amd/csrc/launch.h",
                  "expert_gemms_amd/csrc/l2input.h")


def kernel_sha256():
    """Hash of the GEMM kernel's sources: HBM counters taken from an older
    kernel are not reported."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload, tokens, block_m):
    """HBM bytes per L1 launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
    plain copy of known size), or None when no summary matches the current
    kernel sources and launch."""
    import glob
    sha = kernel_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "l1_gemm_hbm_*.txt"))):
        kv = {}
        with open(path) as f:
            for line in f:
                k, sep, v = line.partition(": ")
                if sep and " " not in k.strip():
                    kv[k.strip()] = v.strip()
        try:
            if (kv.get("workload") == workload and int(kv["tokens"]) == tokens and int(kv["block_m"]) == block_m
                    and kv.get("kernel_sha256") == sha):
                return float(kv["l1_hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            continue
    return None


def elem_bytes(fmt):
    return {"bf16": 2.0, "mxfp8": 1.0, "mxfp4": 0.5, "nvfp4": 0.5}[fmt]


def scale_bytes_per_elem(fmt):
    return {"bf16": 0.0, "mxfp8": 1 / 32, "mxfp4": 1 / 32, "nvfp4": 1 / 16}[fmt]


def build_weights(cfg, device, max_tokens):
    """Weights drawn on the device, quantised by the library's own quantiser
    and transformed to the kernel layout, in a layer sized for max_tokens."""
    import expert_gemms_amd as moe
    from synth import gen_weight_f32_device, gen_w2_input_scale

    fmt = cfg.fmt
    E = cfg.E + cfg.num_shared
    H, I = cfg.H, cfg.I
    vpe = 2 if fmt in ("mxfp4", "nvfp4") else 1
    grp = 16 if fmt == "nvfp4" else 32
    canon = {}
    for name, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
        if fmt == "bf16":
            w = torch.empty((E, N, K), dtype=torch.bfloat16, device=device)
            for e in range(E):
                w[e].copy_(gen_weight_f32_device(cfg, name, e, device))
            canon[name] = w
        else:
            codes = torch.empty((E, N, K // vpe), dtype=torch.uint8, device=device)
            sf = torch.empty((E, N, K // grp), dtype=torch.uint8, device=device)
            gs = torch.empty((E,), dtype=torch.float32, device=device) if fmt == "nvfp4" else None
            for e in range(E):
                src = gen_weight_f32_device(cfg, name, e, device)
                moe.moe_quantize_weights(fmt, 1, N, K, src, codes[e], sf[e],
                                         gs[e:e + 1] if gs is not None else None)
                del src
            canon[name], canon[name + "_sf"] = codes, sf
            if gs is not None:
                canon[name + "_gs"] = gs
    layer = moe.FusedMoE(fmt, H, I, cfg.E, cfg.top_k, num_shared=cfg.num_shared, max_tokens=max_tokens)
    w2_in = torch.from_numpy(gen_w2_input_scale(cfg)) if fmt == "nvfp4" else None
    layer.load_canonical(canon["w13"], canon["w2"], canon.get("w13_sf"), canon.get("w2_sf"),
                         canon.get("w13_gs"), canon.get("w2_gs"), w2_input_scale=w2_in)
    torch.cuda.synchronize()
    return layer, canon


def build_inputs(cfg, T, device):
    """Seeded x (BF16) and routing of T tokens, on the device and the host."""
    from synth import gen_x_bf16, gen_routing
    x = gen_x_bf16(cfg, T).to(device)
    ids, wts = gen_routing(cfg, T)
    return x, ids, wts, torch.from_numpy(ids).to(device), torch.from_numpy(wts).to(device)


def algorithmic(cfg, T, ids):
    """FLOPs and bytes the method itself must compute and move."""
    S = T * (cfg.top_k + cfg.num_shared)
    flops = 6.0 * S * cfg.H * cfg.I
    touched = np.unique(ids[(ids >= 0) & (ids < cfg.E)]).size + cfg.num_shared
    per_expert_elems = 3.0 * cfg.H * cfg.I
    wbytes = touched * per_expert_elems * (elem_bytes(cfg.fmt) + scale_bytes_per_elem(cfg.fmt))
    if cfg.fmt == "nvfp4":
        wbytes += touched * 8
    io = T * cfg.H * 2 * 2 + T * cfg.top_k * 8
    l1_flops = 4.0 * S * cfg.H * cfg.I
    l1_wbytes = touched * 2.0 * cfg.H * cfg.I * (elem_bytes(cfg.fmt) + scale_bytes_per_elem(cfg.fmt))
    return flops, wbytes + io, l1_flops, l1_wbytes, touched


def cpu_baseline(cfg, T, x, ids, wts, canon, n_tok, min_seconds=10.0):
    """The oracle as it stands, on the host cores, over the first n_tok tokens,
    repeated until at least min_seconds have passed (mean time per pass)."""
    from oracle.moe import moe_reference
    from synth import bf16_bits
    from threadpoolctl import threadpool_info

    w = {}
    for k, v in canon.items():
        a = v.cpu().contiguous()
        w[k] = a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else a.numpy()
    xb = bf16_bits(x[:n_tok])
    l2 = 1.0
    if cfg.fmt == "nvfp4":
        from synth import gen_w2_input_scale
        m = float(gen_w2_input_scale(cfg).max())
        l2 = m if m > 0 else 1.0
    passes, t0 = 0, time.perf_counter()
    while True:
        moe_reference(cfg.fmt, xb, ids[:n_tok], wts[:n_tok], w, num_shared=cfg.num_shared,
                      l2_activation_scale=l2)
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = (time.perf_counter() - t0) / passes
    S = n_tok * (cfg.top_k + cfg.num_shared)
    flops = 6.0 * S * cfg.H * cfg.I
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    touched = np.unique(ids[:n_tok][(ids[:n_tok] >= 0) & (ids[:n_tok] < cfg.E)]).size + cfg.num_shared
    host = host_cpu()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(min(threads, host["usable_cpus"])),
            "kind": "oracle", "blas_threads": int(threads), "physical_cores": host["physical_cores"],
            "usable_cpus": host["usable_cpus"], "cpu_model": host["model"],
            "sample": f"first {n_tok} of {T} tokens of the same workload ({S} slots, {touched} experts "
                      f"dequantised per pass); {passes} pass(es), {dt:.2f} s per pass"}


def host_cpu():
    """CPU model, physical cores of the host and CPUs this process may use."""
    model, cores = "unknown", set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name":
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return {"model": model, "physical_cores": len(cores) or None, "usable_cpus": usable}


def default_cpu_tokens(cfg, T):
    """Oracle sample: every token when the experts are few and large (the
    dequantisation is shared by many rows), else a handful of tokens (each
    touched expert costs a full fp64 dequantisation)."""
    return min(T, 4096) if cfg.E <= 16 else min(T, 4)


# Router top-k settings per workload: (scoring, bias, groups, kept groups,
# renormalise, scaling) -- DeepSeek-V3's sigmoid scores with correction bias
# and 8 groups of which 4 are kept; softmax top-k elsewhere.
ROUTE_STYLE = {
    "tiny_bf16": ("softmax", False, 1, 1, True, 1.0),
    "mixtral_bf16": ("softmax", False, 1, 1, True, 1.0),
    "dsv3_mxfp8": ("sigmoid", True, 8, 4, True, 2.5),
    "decode_mxfp4": ("softmax", False, 1, 1, True, 1.0),
    "nvfp4_zipf": ("softmax", False, 1, 1, True, 1.0),
}


def route_bench(args, cfg, T):
    """Router top-k on [T, E] float32 logits: tokens/s, HBM roofline, and the
    oracle on the host for comparison."""
    import expert_gemms_amd as moe
    from oracle.routing import route_reference

    scoring, use_bias, G, TG, renorm, scaling = ROUTE_STYLE[cfg.name]
    E, k = cfg.E, cfg.top_k
    rng = np.random.default_rng(cfg.cfg_id)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32) if use_bias else None
    dl = torch.from_numpy(logits).cuda()
    db = None if bias is None else torch.from_numpy(bias).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    run = lambda: moe.moe_route(T, E, k, dl, ids, wts, bias=db, scoring=scoring, num_groups=G, topk_groups=TG,
                                renormalize=renorm, routed_scaling_factor=scaling)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = T * E * 4 + T * k * 8 + (E * 4 if use_bias else 0)
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        n = min(T, 8192)
        t0, passes = time.perf_counter(), 0
        while time.perf_counter() - t0 < 10.0:
            route_reference(logits[:n].astype(np.float64), k, scoring=scoring,
                            bias=None if bias is None else bias.astype(np.float64), num_groups=G,
                            topk_groups=TG, renormalize=renorm, scaling=scaling)
            passes += 1
        dt = (time.perf_counter() - t0) / passes
        cpu = {"value": round(n / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} of {T} tokens; {passes} pass(es), {dt:.3f} s per pass"}
    rec = {"metric": "router top-k tokens/s", "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded N(0,1) router logits)",
           "config": {"workload": cfg.name + " routing", "tokens": T, "experts": E, "top_k": k,
                      "scoring": scoring, "bias": use_bias, "groups": G, "kept_groups": TG},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "router top-k"},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)
    return 0


def time_workload(args, cfg, T, flush_mb, layer, canon, min_cpu_seconds):
    """One workload: warm-up, K timed steps, per-step kernel times, the
    percentiles, a graph replay, the roofline of the L1 GEMM and the oracle
    beside it.  Returns the record."""
    import expert_gemms_amd as moe

    device = torch.device("cuda:0")
    x, ids, wts, ids_d, wts_d = build_inputs(cfg, T, device)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=device)
    stream = torch.cuda.current_stream()
    flush = torch.ones(flush_mb * (1 << 18), dtype=torch.int32, device=device) if flush_mb else None
    flush_sink = torch.zeros((), dtype=torch.int64, device=device)

    def evict():
        flush_sink.add_(flush.sum())

    nsteps = len(moe._lib.STEPS)

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nsteps)]
        for e in evs:
            e.record(stream)          # creates the underlying hipEvent
        return evs

    fwd = lambda: layer.forward(x, ids_d, wts_d, out=out, block_m=args.block_m)
    for _ in range(args.warmup):
        if flush is not None:
            evict()
        fwd()
    torch.cuda.synchronize()

    # timed: K plain steps (with a flush, each step is timed on its own so
    # the flush stays outside)
    wall0 = time.perf_counter()
    if flush is None:
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for i in range(args.steps):
            fwd()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_per_step = t_start.elapsed_time(t_end) / args.steps
    else:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            evict()
            evs[i][0].record(stream)
            fwd()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ms_per_step = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    wall = time.perf_counter() - wall0

    # per-step device times (the library records HIP events around each step
    # on its launch stream), from K more steps
    step_events = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        if flush is not None:
            evict()
        layer.forward(x, ids_d, wts_d, out=out, block_m=args.block_m, step_events=step_events[i])
    torch.cuda.synchronize()
    per_step = {name: float(np.mean([ev[2 * j].elapsed_time(ev[2 * j + 1]) for ev in step_events]))
                for j, name in enumerate(moe._lib.STEPS)}
    # spread of the step time: K more steps, each between one pair of events
    # (no events inside the step; each pair adds a few microseconds, which
    # shows at decode sizes)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        if flush is not None:
            evict()
        pairs[i][0].record(stream)
        fwd()
        pairs[i][1].record(stream)
    torch.cuda.synchronize()
    totals = [a.elapsed_time(b) for a, b in pairs]
    step_pct = {q: round(float(np.percentile(totals, q)), 4) for q in (10, 50, 90)}

    # secondary: the step captured once in a HIP graph and replayed (launch
    # overhead removed); the replay's output is checked against the eager one
    graph_ms = None
    if not args.no_graph:
        ref_out = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fwd()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref_out):
            raise RuntimeError("graph replay differs from the eager step")
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del g

    flops, hbm_bytes, l1_flops, l1_wbytes, touched = algorithmic(cfg, T, ids)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbs = hbm_bytes / (ms_per_step * 1e-3) / 1e9
    l1_ms = per_step["l1"]
    peak = PEAK_TFLOPS[cfg.fmt]
    prefill = l1_flops / l1_wbytes > peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if prefill:
        achieved = l1_flops / (l1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None, "kernel": "L1 grouped GEMM"}
        if cfg.fmt == "nvfp4":
            roof["peak_note"] = "FP16 MFMA (exactly dequantised NVFP4 operands)"
            roof["frac_of_fp4_peak"] = round(achieved / PEAK_FP4_TFLOPS, 4)
    else:
        achieved = l1_wbytes / (l1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "L1 grouped GEMM"}

    bm = args.block_m or layer_block_m(cfg, T)
    traffic = profiled_traffic(cfg.name, T, bm)
    roof["traffic"] = None if traffic is None else round(traffic / 1e9, 4)
    roof["traffic_unit"] = "GB per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["algorithmic_per_launch"] = (round(l1_flops / 1e12, 4) if prefill else round(l1_wbytes / 1e9, 4))
    roof["algorithmic_unit"] = "TFLOP" if prefill else "GB"

    cpu = None
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens or default_cpu_tokens(cfg, T)
        cpu = cpu_baseline(cfg, T, x, ids, wts, canon, n_tok, min_seconds=min_cpu_seconds)

    S = T * (cfg.top_k + cfg.num_shared)
    mfma_frac = tflops / peak
    rec = {
        "metric": "MoE-layer TFLOP/s (HBM GB/s alongside; fraction of MI355X peak) per format",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.fmt,
        "data": "synthetic (seeded; random-init weights of the named shape)",
        "config": {"workload": cfg.name, "format": cfg.fmt, "tokens": T, "hidden": cfg.H, "inter": cfg.I,
                   "experts": cfg.E, "shared": cfg.num_shared, "top_k": cfg.top_k, "slots": S,
                   "touched_experts": int(touched), "block_m": bm, "flush_mb": flush_mb},
        "hbm_gbps": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "mfma_frac": round(mfma_frac, 4),
        # the step's roofline time t* = max(F / MFMA peak, B / HBM peak) and
        # t* over the measured time (= the larger of the two fractions)
        "t_star_ms": round(max(mfma_frac, gbs / PEAK_HBM_GBS) * ms_per_step, 4),
        "t_star_over_t": round(max(mfma_frac, gbs / PEAK_HBM_GBS), 4),
        "step_ms": {k: round(v, 4) for k, v in per_step.items()},
        "step_ms_p10_p50_p90": [step_pct[10], step_pct[50], step_pct[90]],
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "wall_s": round(wall, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if cfg.fmt == "nvfp4":
        rec["mfma_frac_of_fp4_peak"] = round(tflops / PEAK_FP4_TFLOPS, 4)
    del out, flush
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported by this build "
              "(the layer's expert-parallel path across GPUs is not built)", file=sys.stderr)
        return 2
    if args.copy_mb:
        return copy_calibration(args.copy_mb)
    from synth import CONFIGS

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.config is not None:
        cfg = CONFIGS[args.config]
        T = args.tokens if args.tokens is not None else cfg.T
        if args.route:
            return route_bench(args, cfg, T)
        layer, canon = build_weights(cfg, device, T)
        rec = time_workload(args, cfg, T, args.flush_mb, layer, canon, 10.0)
        print(json.dumps(rec), flush=True)
        return 0

    # every workload; the weights of one workload are built once for all its
    # token counts and freed before the next workload
    plan = [HEADLINE] + SUB_WORKLOADS
    recs, built = [], (None, None, None)
    for i, (name, tokens, flush_mb) in enumerate(plan):
        cfg = CONFIGS[name]
        T = tokens if tokens is not None else cfg.T
        if built[0] != name:
            built = (None, None, None)
            torch.cuda.empty_cache()
            max_t = max((t if t is not None else cfg.T) for n, t, _ in plan if n == name)
            layer, canon = build_weights(cfg, device, max_t)
            built = (name, layer, canon)
        _, layer, canon = built
        print(f"bench: {name} T={T}", file=sys.stderr, flush=True)
        recs.append(time_workload(args, cfg, T, flush_mb, layer, canon, 10.0 if i == 0 else 5.0))
    head = recs[0]
    head["workloads"] = recs[1:]
    print(json.dumps(head), flush=True)
    return 0


def layer_block_m(cfg, T):
    import expert_gemms_amd as moe
    return moe.moe_get_block_m(T, cfg.E, cfg.num_shared, cfg.top_k, cfg.fmt)


if __name__ == "__main__":
    sys.exit(main())
