#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

One step = router top-k + the fused MoE FFN layer (alignment, GEMM1 with
SiLU(C1)*C2, GEMM2, combine) over one batch of seeded synthetic input, all
inputs and (prepacked) weights resident in HBM before timing starts.
Consecutive steps cycle through R different router-logit batches so every
step routes to a different expert set (weights are streamed from HBM, not
re-read from the 256 MB Infinity Cache).

Prints ONE JSON line: tokens/s of the workload, the roofline of the dominant
kernel (GEMM1: HBM bytes for decode / INT8, bf16-MFMA FLOPs for FP8 prefill)
from per-kernel HIP events, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload c2]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM TB/s and prefill MFMA TFLOP/s vs peak"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
MFMA_I8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm1_model(cfg, n_distinct):
    """Algorithmic bytes and FLOPs of one GEMM1 launch (gate/up GEMM + SiLU):
    the weights (and scales) of every expert the step routes to, read once;
    the token rows read once; the intermediate written once."""
    from mixture_experts_ffn_topk_amd import synth
    elem = 2 if cfg.wdtype == synth.WDTYPE_BF16 else 1
    w13 = cfg.H * 2 * cfg.I * elem
    if cfg.wdtype == synth.WDTYPE_FP8:
        w13 += 4 * (cfg.H // 128) * (2 * cfg.I // 128)
    elif cfg.wdtype == synth.WDTYPE_INT8:
        w13 += 4 * 2 * cfg.I
    experts = n_distinct + (1 if cfg.shared else 0)
    rows = cfg.T * cfg.k + (cfg.T if cfg.shared else 0)
    xbytes = cfg.T * cfg.H * (1 if cfg.wdtype == synth.WDTYPE_INT8 else 2)
    nbytes = experts * w13 + xbytes + rows * cfg.I * 2
    flops = 2.0 * rows * cfg.H * 2 * cfg.I
    return nbytes, flops


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from a committed
    rocprofv3 counter summary under profiles/ (FETCH_SIZE + WRITE_SIZE passes
    scaled by a plain-copy calibration), or None when there is none or the
    kernel's sources changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))):
        fields = {}
        for line in open(path):
            key, sep, val = line.strip().partition(": ")
            if sep and key in ("workload", "kernel", "traffic_bytes_per_launch", "kernel_sources",
                               "kernel_sources_sha256"):
                fields[key] = val.strip()
        if fields.get("workload") != workload or fields.get("kernel") != kernel:
            continue
        h = hashlib.sha256()
        try:
            for f in fields["kernel_sources"].split():
                with open(os.path.join(ROOT, f), "rb") as fh:
                    h.update(fh.read())
        except (KeyError, OSError):
            return None
        if h.hexdigest() != fields.get("kernel_sources_sha256"):
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    return None


def host_cpu():
    """Logical CPUs visible to this process and the CPU model name (for the
    oracle's context; the oracle itself runs on one thread)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 0
    return {"nproc": n, "model": model}


def cpu_baseline(inp, budget_s=15.0):
    """The oracle (single-threaded C, fp64) on the first n tokens of the same
    workload: its own top-k, then the per-token loop.  n is sized so the run
    takes about budget_s seconds.  -> (tokens/s, n tokens, seconds)."""
    import numpy as np
    import torch

    import oracle
    cfg = inp.cfg
    lg = inp.logits.cpu()
    x = inp.x.cpu()

    def run(n):
        t0 = time.perf_counter()
        w, ids = oracle.topk(lg[:n], cfg.k, cfg.score, cfg.renorm)
        t_route = time.perf_counter() - t0
        used = sorted(set(ids.reshape(-1).tolist()))
        remap = np.zeros(cfg.E, np.int32)
        remap[used] = np.arange(len(used))
        sel = torch.tensor(used, device=inp.w13.device)
        pick = (lambda w: w.view(torch.int16).index_select(0, sel).view(torch.uint16).cpu()
                if w.dtype == torch.uint16 else w.index_select(0, sel).cpu())
        w13, w2 = pick(inp.w13), pick(inp.w2)
        s13 = None if inp.w13_scale is None else inp.w13_scale.index_select(0, sel).cpu()
        s2 = None if inp.w2_scale is None else inp.w2_scale.index_select(0, sel).cpu()
        c = (lambda t: None if t is None else t.cpu())
        t1 = time.perf_counter()
        oracle.moe(cfg.wdtype, x[:n], w13, s13, w2, s2, w.astype(np.float32), remap[ids],
                   c(inp.sh13), c(inp.sh13_scale), c(inp.sh2), c(inp.sh2_scale))
        return t_route + time.perf_counter() - t1

    t1 = run(1)
    n = int(max(1, min(cfg.T, budget_s / max(t1, 1e-6))))
    t = run(n) if n > 1 else t1
    return n / t, n, t


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200 for decode-sized T*k/E <= 8, else 50)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2",
                    help="c1, c2 (default: DeepSeek-R1-shaped FP8 decode, T=4), c3, c4, "
                         "c5_T1, c5_T32, c5_T2048")
    ap.add_argument("--routings", type=int, default=16, help="router-logit batches cycled")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the workload, run one plain device copy of this many MiB "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the layer runs and is measured on one GPU only (asked for --gpus "
              f"{args.gpus}, WORLD_SIZE={world}); sharding over several GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_ffn_topk_amd import _lib as moe
    from mixture_experts_ffn_topk_amd import synth

    if args.workload not in synth.CONFIGS:
        sys.exit(f"unknown workload {args.workload}")
    cfg = synth.CONFIGS[args.workload]
    if args.steps is None:
        args.steps = 200 if cfg.T * cfg.k / cfg.E <= 8.0 else 50
    dev = "cuda:0"
    torch.cuda.set_device(0)
    path = {"auto": moe.PATH_AUTO, "decode": moe.PATH_DECODE, "prefill": moe.PATH_PREFILL}[args.path]

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes read + {n} bytes written by one copy kernel")
        del src, dst

    t0 = time.time()
    inp = synth.draw_inputs(cfg, dev)
    layer = moe.MoELayer(inp, path=path, split_k=args.split_k)
    R = max(1, args.routings)
    logits = [inp.logits] + [synth.draw_logits(cfg, dev, seed=cfg.seed + 7919 * r)
                             for r in range(1, R)]
    x = inp.x
    distinct = []
    for lg in logits:
        _, ids = layer.route(lg)
        distinct.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: inputs ready in {time.time() - t0:.1f}s; distinct experts per "
        f"routing {distinct}")

    for i in range(args.warmup):
        layer.step(logits[i % R], x)
    torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        layer.step(logits[i % R], x)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    tok_s = cfg.T / (ms / 1e3)
    log(f"[bench] {args.steps} steps: {ms * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} "
        f"us/step), {tok_s:.1f} tokens/s")

    # small batches: the same steps as one captured HIP graph (R steps per
    # graph, one per routing), replayed; launch overhead drops out
    graph = None
    if cfg.T <= 64:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(R):
                layer.step(logits[i], x)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                layer.step(logits[i], x)
        torch.cuda.synchronize()
        reps = max(1, args.steps // R)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / (reps * R)
        graph = {"ms_per_step": round(gms, 5), "tokens_per_s": round(cfg.T / (gms / 1e3), 2),
                 "steps": reps * R}
        log(f"[bench] graph-launched: {gms * 1e3:.1f} us/step, {cfg.T / (gms / 1e3):.1f} tokens/s")
        del g

    # per-kernel durations: same steps again with events around every kernel
    moe.profile_enable(True)
    nprof = max(R, min(args.steps, 4 * R))
    for i in range(nprof):
        layer.step(logits[i % R], x)
    torch.cuda.synchronize()
    prof = moe.profile_collect()
    moe.profile_enable(False)
    kern = {k: (v[0] / v[1]) * 1e3 for k, v in prof.items()}  # us per launch
    log("[bench] per-kernel us: " + ", ".join(f"{k}={v:.1f}" for k, v in kern.items()))

    avg_distinct = sum(distinct[i % R] for i in range(nprof)) / nprof
    nbytes, flops = gemm1_model(cfg, avg_distinct)
    g1 = kern.get("gemm1", float("nan"))
    prefill_fp = cfg.wdtype != synth.WDTYPE_INT8 and layer.w13 is not None and \
        cfg.T * cfg.k / cfg.E > 8.0 and path != moe.PATH_DECODE
    if prefill_fp:
        achieved = flops / (g1 * 1e-6) / 1e12
        roof = {"kernel": "gemm1 (grouped gate/up GEMM + SiLU)", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                "algorithmic_flops_per_launch": flops, "avg_launch_us": round(g1, 2)}
    else:
        achieved = nbytes / (g1 * 1e-6) / 1e9
        roof = {"kernel": "gemm1 (grouped gate/up GEMM + SiLU)", "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(cfg.name, "gemm1"),
                "algorithmic_bytes_per_launch": int(nbytes), "avg_launch_us": round(g1, 2)}
    # whole layer: both weight matrices of every routed expert, logits, x and out
    layer_bytes = (avg_distinct + (1 if cfg.shared else 0)) * synth.bytes_per_expert(cfg) + \
        cfg.T * cfg.E * 4 + 2 * cfg.T * cfg.H * 2
    res = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if cfg.wdtype == synth.WDTYPE_INT8 else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "top_k": cfg.k, "shared_expert": cfg.shared,
                   "weights": {0: "bf16", 1: "fp8_e4m3fn_128x128", 2: "int8_per_channel"}[cfg.wdtype],
                   "routing": cfg.routing, "routings_cycled": R,
                   "avg_distinct_experts": avg_distinct, "path": args.path,
                   "parallelism": "1 GPU"},
        "roofline": roof,
        "kernel_us": {k: round(v, 2) for k, v in kern.items()},
        "layer_algorithmic_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
    }
    if graph is not None:
        res["graph_launched"] = graph
    if not args.no_cpu_baseline:
        tps, n, secs = cpu_baseline(inp, args.cpu_budget)
        res["cpu_baseline"] = {"value": round(tps, 4), "unit": "tokens/s", "cores": 1,
                               "kind": "oracle", "host": host_cpu(),
                               "sample": f"first {n} of {cfg.T} tokens of the same workload "
                                         f"(oracle top-k + per-token fp64 FFN loop), "
                                         f"{secs:.1f} s, single thread"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
