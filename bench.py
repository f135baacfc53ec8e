#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

One step = router top-k + the fused MoE FFN layer (alignment, GEMM1 with
SiLU(C1)*C2, GEMM2, combine) over one batch of seeded synthetic input, all
inputs and (prepacked) weights resident in HBM before timing starts.
Consecutive steps cycle through R different router-logit batches so every
step routes to a different expert set (weights are streamed from HBM, not
re-read from the 256 MB Infinity Cache).

Prints ONE JSON line.  Its headline is the largest single-GPU workload, the
DeepSeek-R1-shaped FP8 prefill of 4096 tokens (c4): tokens/s over exactly
--steps timed steps, the roofline of its dominant kernel (GEMM1, bf16-rate
MFMA FLOPs from per-kernel HIP events), and the CPU oracle timed on a bounded
sample on all host cores and on one.  The other workloads (c1, c2, c3, c5 at
T = 1 / 32 / 2048) follow as sub-records under "workloads", each with its
tokens/s, graph-launched time (T <= 64) and its GEMMs' roofline fractions.

    python bench.py [--steps K] [--warmup W] [--workload c4] [--sub c1,c2,...|none]
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM TB/s and prefill MFMA TFLOP/s vs peak"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
MFMA_I8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA
MFMA_F8_PEAK_TFS = 5000.0    # MI355X dense fp8 MFMA
# sub-records that are a workload run with an option: name -> (workload, FP8 activations)
VARIANTS = {"c4_fp8_act": ("c4", 1)}
# c2_int4: the DeepSeek-R1-shaped decode batch with INT4 weight-only experts
ALL = ["c1", "c2", "c3", "c4", "c4_fp8_act", "c5_T1", "c5_T32", "c5_T2048", "c2_int4"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_model(cfg, n_distinct, which):
    """Algorithmic bytes and FLOPs of one launch of GEMM1 (gate/up + SiLU) or
    GEMM2 (down): the weights (and scales) of every expert the step routes to,
    read once; the GEMM's input rows read once (GEMM1: the token rows, bf16 or
    INT8; GEMM2: the intermediate rows, bf16 or INT8 + a row scale); its
    output rows written once (GEMM1: bf16 intermediate; GEMM2: bf16 y rows)."""
    from mixture_experts_ffn_topk_amd import synth
    i8 = cfg.wdtype == synth.WDTYPE_INT8
    elem = 2 if cfg.wdtype == synth.WDTYPE_BF16 else 1
    K, N = (cfg.H, 2 * cfg.I) if which == 1 else (cfg.I, cfg.H)
    w = K * N * elem
    if cfg.wdtype == synth.WDTYPE_FP8:
        w += 4 * (K // 128) * (N // 128)
    elif i8:
        w += 4 * N
    elif cfg.wdtype == synth.WDTYPE_INT4:  # two codes per byte, a scale per column and 128 rows
        w = K * N // 2 + 4 * (K // 128) * N
    experts = n_distinct + (1 if cfg.shared else 0)
    rows = cfg.T * cfg.k + (cfg.T if cfg.shared else 0)
    if which == 1:
        a_bytes = cfg.T * cfg.H * (1 if i8 else 2) + (4 * cfg.T if i8 else 0)
        o_bytes = rows * cfg.I * 2
    else:
        a_bytes = rows * cfg.I * (1 if i8 else 2) + (4 * rows if i8 else 0)
        o_bytes = rows * cfg.H * 2
    return experts * w + a_bytes + o_bytes, 2.0 * rows * K * N


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
    """Logical CPUs this process may run on and the CPU model name."""
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


def cpu_baseline(inp, budget_s=10.0, one_thread_budget_s=4.0, repeats=1):
    """The oracle as it stands (plain C, fp64) on the first n tokens of the
    same workload: its own top-k, then the per-token layer loop, token shards
    on all host threads; then the same on one thread over a smaller sample.
    n is sized from a one-token probe so each run takes about its budget.
    repeats > 1 takes the median of that many runs."""
    import numpy as np
    import torch

    import oracle
    cfg = inp.cfg
    lg = inp.logits.cpu()
    x = inp.x.cpu()
    c = (lambda t: None if t is None else t.cpu())
    w13, w2 = c(inp.w13), c(inp.w2)
    s13, s2 = c(inp.w13_scale), c(inp.w2_scale)
    sh = (c(inp.sh13), c(inp.sh13_scale), c(inp.sh2), c(inp.sh2_scale))

    def run(n, threads):
        t0 = time.perf_counter()
        w, ids = oracle.topk(lg[:n], cfg.k, cfg.score, cfg.renorm)
        oracle.moe(cfg.wdtype, x[:n], w13, s13, w2, s2, w.astype(np.float32), ids, *sh,
                   threads=threads)
        return time.perf_counter() - t0

    nthr = oracle.host_threads()
    t1 = run(1, 1)
    res = {}
    for key, threads, budget in (("all", nthr, budget_s), ("one", 1, one_thread_budget_s)):
        n = int(max(1, min(cfg.T, budget * threads / max(t1, 1e-6))))
        times = [run(n, threads) for _ in range(repeats)]
        t = statistics.median(times)
        res[key] = (n / t, n, t, min(threads, n))
    return res


def run_workload(name, inp, layer, args, steps, R, prepack_ms, fp8_act=0):
    """Time one workload: warm-up, exactly `steps` back-to-back steps between
    HIP events on the stream, the graph-launched form (T <= 64), then a
    second pass with events around every library kernel for the rooflines."""
    import numpy as np
    import torch

    from mixture_experts_ffn_topk_amd import _lib as moe
    from mixture_experts_ffn_topk_amd import synth
    cfg = inp.cfg
    dev = inp.x.device
    logits = [inp.logits] + [synth.draw_logits(cfg, dev, seed=cfg.seed + 7919 * r)
                             for r in range(1, R)]
    x = inp.x
    distinct, counts = [], []
    for lg in logits:
        _, ids = layer.route(lg)
        distinct.append(int(torch.unique(ids).numel()))
        counts.append(torch.bincount(ids.reshape(-1).long(), minlength=cfg.E).cpu().numpy())
    torch.cuda.synchronize()
    log(f"[bench] {name} ({cfg.name}): distinct experts per routing {distinct}")

    for i in range(args.warmup):
        layer.step(logits[i % R], x)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        layer.step(logits[i % R], x)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / steps
    tok_s = cfg.T / (ms / 1e3)
    log(f"[bench] {name}: {steps} steps: {ms * 1e3:.1f} us/step (wall "
        f"{wall / steps * 1e6:.1f} us/step), {tok_s:.1f} tokens/s")

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
        reps = max(1, steps // R)
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
        log(f"[bench] {name}: graph-launched {gms * 1e3:.1f} us/step")
        del g

    moe.profile_enable(True)
    nprof = max(R, min(steps, 4 * R))
    for i in range(nprof):
        layer.step(logits[i % R], x)
    torch.cuda.synchronize()
    prof = moe.profile_collect()
    moe.profile_enable(False)
    kern = {k: (v[0] / v[1]) * 1e3 for k, v in prof.items()}  # us per launch
    log(f"[bench] {name}: per-kernel us: " + ", ".join(f"{k}={v:.1f}" for k, v in kern.items()))

    avg_distinct = sum(distinct[i % R] for i in range(nprof)) / nprof
    prefill = cfg.T * cfg.k / cfg.E > 8.0
    i8 = cfg.wdtype == synth.WDTYPE_INT8
    roofs = {}
    for which, key in ((1, "gemm1"), (2, "gemm2")):
        nbytes, flops = gemm_model(cfg, avg_distinct, which)
        us = kern.get(key, float("nan"))
        gbs = nbytes / (us * 1e-6) / 1e9
        if prefill and not i8:
            # FP8 / BF16 weights on the MFMA tile kernels: bf16-rate products
            # (FP8 activations: one FP8 MFMA per product, the FP8 peak)
            peak = MFMA_F8_PEAK_TFS if fp8_act else MFMA_BF16_PEAK_TFS
            ach = flops / (us * 1e-6) / 1e12
            r = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                 "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                 "algorithmic_flops_per_launch": flops, "hbm_gbs": round(gbs, 1)}
        else:
            # decode, and INT8 prefill (arithmetic intensity below the int8 ridge)
            r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes_per_launch": int(nbytes)}
            if prefill:
                tops = flops / (us * 1e-6) / 1e12
                r["mfma_int8_tops"] = round(tops, 1)
                r["mfma_int8_frac"] = round(tops / MFMA_I8_PEAK_TOPS, 4)
        r["avg_launch_us"] = round(us, 2)
        r["traffic"] = measured_traffic(cfg.name + ("+fp8_act" if fp8_act else ""), key)
        roofs[key] = r
    layer_bytes = (avg_distinct + (1 if cfg.shared else 0)) * synth.bytes_per_expert(cfg) + \
        cfg.T * cfg.E * 4 + 2 * cfg.T * cfg.H * 2
    rec = {
        "workload": cfg.name, "T": cfg.T, "tokens_per_s": round(tok_s, 2),
        "fp8_activations": bool(fp8_act),
        "ms_per_step": round(ms, 5), "steps": steps,
        "graph_launched": graph,
        "kernel_us": {k: round(v, 2) for k, v in kern.items()},
        "roofline": roofs,
        "layer_algorithmic_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
        "avg_distinct_experts": avg_distinct,
        # one-time weight prepack of the whole layer (w13, w2, shared), not timed
        "prepack_ms": round(prepack_ms, 3) if prepack_ms is not None else None,
    }
    # expert load of the seeded routing (the workload's own logits): balance =
    # mean / max of the per-expert pair counts, and of the rows after padding
    # to the 16-row alignment block (the grouped GEMMs' work)
    c0 = counts[0].astype(np.int64)
    padded = (c0 + 15) // 16 * 16
    bal = {"pairs_mean_over_max": round(float(c0.mean() / c0.max()), 4),
           "padded_rows_mean_over_max": round(float(padded.mean() / padded.max()), 4),
           "max_pairs": int(c0.max()), "experts_used": int((c0 > 0).sum())}
    if cfg.routing == "zipf" or cfg.T >= 64:
        edges = [0, 1, 2, 4, 8, 16, 32, 64, 128, 256, 1 << 30]
        hist = {}
        for lo, hi in zip(edges[:-1], edges[1:]):
            n = int(((c0 >= lo) & (c0 < hi)).sum())
            if n:
                hist[f"{lo}" if hi == lo + 1 else f"{lo}-{hi - 1}" if hi < 1 << 30 else f">={lo}"] = n
        bal["histogram_experts_by_pairs"] = hist
        bal["top8_pairs"] = sorted(c0.tolist(), reverse=True)[:8]
        bal["mean_over_max_all_routings"] = round(
            float(np.mean([c.mean() / c.max() for c in counts])), 4)
    rec["expert_load"] = bal
    return rec, tok_s, ms, avg_distinct


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4", help="headline workload (default c4)")
    ap.add_argument("--sub", default="others",
                    help="comma list of other workloads for sub-records, 'others' (default: "
                         "every other workload) or 'none'")
    ap.add_argument("--sub-steps", type=int, default=200,
                    help="timed steps of each sub-record workload (at least --steps)")
    ap.add_argument("--routings", type=int, default=16, help="router-logit batches cycled")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of the all-core oracle run (the one-thread run takes ~0.4x)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the workloads, run one plain device copy of this many MiB "
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
    def cfg_of(w):
        if w in VARIANTS:
            return synth.CONFIGS[VARIANTS[w][0]]
        return synth.EXTRA_CONFIGS[w] if w in synth.EXTRA_CONFIGS else synth.CONFIGS.get(w)
    if args.sub == "none":
        subs = []
    elif args.sub == "others":
        subs = [w for w in ALL if w != args.workload]
    else:
        subs = [w for w in args.sub.split(",") if w and w != args.workload]
    for w in subs:
        if cfg_of(w) is None:
            sys.exit(f"unknown workload {w}")
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

    # workloads that share a weight set run back to back on one packed copy
    order = [args.workload] + subs
    groups = {}
    for w in order:
        c = cfg_of(w)
        groups.setdefault((c.wdtype, c.H, c.I, c.E, c.shared), []).append(w)
    head = None
    subrec = {}
    for key, names in groups.items():
        t0 = time.time()
        base = cfg_of(names[0])
        inp0 = synth.draw_inputs(base, dev)
        torch.cuda.synchronize()
        log(f"[bench] weights of {names} drawn in {time.time() - t0:.1f}s")
        packed = None
        group_prepack_ms = None
        for w in names:
            cfg = cfg_of(w)
            fp8_act = VARIANTS[w][1] if w in VARIANTS else 0
            inp = synth.MoEInputs(cfg, synth.draw_logits(cfg, dev), synth.draw_x(cfg, dev),
                                  inp0.w13, inp0.w13_scale, inp0.w2, inp0.w2_scale, inp0.sh13,
                                  inp0.sh13_scale, inp0.sh2, inp0.sh2_scale)
            prepack_ms = None
            if packed is None:
                torch.cuda.synchronize()
                p0 = torch.cuda.Event(enable_timing=True)
                p1 = torch.cuda.Event(enable_timing=True)
                p0.record()
                layer = moe.MoELayer(inp, path=path, split_k=args.split_k, fp8_act=fp8_act)
                p1.record()
                torch.cuda.synchronize()
                prepack_ms = p0.elapsed_time(p1)
                packed = layer
            else:
                layer = moe.MoELayer(inp, path=path, split_k=args.split_k, packed_from=packed,
                                     fp8_act=fp8_act)
            is_head = w == args.workload
            decode_sized = cfg.T * cfg.k / cfg.E <= 8.0
            steps = args.steps if is_head else max(args.steps, args.sub_steps if decode_sized
                                                    else min(args.sub_steps, 50))
            if prepack_ms is not None:
                group_prepack_ms = prepack_ms
            rec, tok_s, ms, avg_distinct = run_workload(w, inp, layer, args, steps,
                                                        max(1, args.routings), group_prepack_ms,
                                                        fp8_act)
            if is_head:
                cpu = None
                if not args.no_cpu_baseline:
                    res = cpu_baseline(inp, args.cpu_budget, 0.4 * args.cpu_budget,
                                       repeats=1 if not decode_sized else 3)
                    (v_all, n_all, t_all, c_all), (v_one, n_one, t_one, _) = res["all"], res["one"]
                    cpu = {"value": round(v_all, 4), "unit": "tokens/s", "cores": c_all,
                           "kind": "oracle", "host": host_cpu(),
                           "sample": f"first {n_all} of {cfg.T} tokens of the same workload "
                                     f"(oracle top-k + per-token fp64 layer loop, token shards "
                                     f"on {c_all} threads), {t_all:.1f} s"
                                     + (", median of 3" if decode_sized else ""),
                           "one_thread": {"value": round(v_one, 4), "unit": "tokens/s",
                                          "sample": f"first {n_one} tokens, {t_one:.1f} s"}}
                    log(f"[bench] oracle: {v_all:.3f} tokens/s on {c_all} threads, "
                        f"{v_one:.3f} on one")
                head = (rec, tok_s, ms, avg_distinct, cfg, steps, cpu)
            else:
                subrec[w] = rec
            del layer
        del packed, inp0
        torch.cuda.empty_cache()

    rec, tok_s, ms, avg_distinct, cfg, steps, cpu = head
    r1 = dict(rec["roofline"]["gemm1"])
    r1["kernel"] = "gemm1 (grouped gate/up GEMM + SiLU)"
    res = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if cfg.wdtype == synth.WDTYPE_INT8 else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "top_k": cfg.k, "shared_expert": cfg.shared,
                   "weights": {0: "bf16", 1: "fp8_e4m3fn_128x128", 2: "int8_per_channel",
                               3: "int4_group128"}[cfg.wdtype],
                   "routing": cfg.routing, "routings_cycled": max(1, args.routings),
                   "avg_distinct_experts": avg_distinct, "path": args.path,
                   "parallelism": "1 GPU"},
        "roofline": r1,
        "gemm2_roofline": rec["roofline"]["gemm2"],
        "kernel_us": rec["kernel_us"],
        "layer_algorithmic_gbs": rec["layer_algorithmic_gbs"],
        "prepack_ms": rec["prepack_ms"],
        "expert_load": rec["expert_load"],
    }
    if rec["graph_launched"] is not None:
        res["graph_launched"] = rec["graph_launched"]
    if cpu is not None:
        res["cpu_baseline"] = cpu
    res["workloads"] = subrec
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
