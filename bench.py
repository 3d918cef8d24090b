"""Benchmark of the fused int4 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--m 9] [--workload decode]

A step is one call of the whole layer (route, gate+up, down, combine) on one
batch of M tokens.  Each step gets its own seeded activations and router
logits (uploaded before timing), so consecutive steps touch different
experts and the weight stream is not served from the 256 MB last-level
cache.  Inputs are resident in HBM when the timed region starts.

Prints one JSON line: throughput in tokens/s for the workload, the
roofline of the dominant kernel (gate+up) from HIP events on the stream the
kernels run on, and the CPU oracle timed on the host's cores on a bounded
sample.  The layer's shapes are those of the M-sweep in "The MoE Throughput
Lever: Quantifying the INT4 Marlin GEMM on Blackwell PRO 6000" (section
"The Benchmark: What Was Measured"); its per-M figures for one RTX PRO 6000
Blackwell are reported as context (vs_baseline), not as a target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "MoE layer µs/call & tokens/s vs M (1..4096); % HBM BW / % bf16 MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, published
# ms/call of the INT4 Marlin MoE on one RTX PRO 6000 Blackwell, same layer
PAGE_MS_PER_CALL = {1: 0.151, 9: 1.18, 90: 5.19, 256: 7.02, 512: 7.01, 1024: 7.02}
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_mixture_experts_top_amd", "csrc", f) for f in ("qmoe.hip", "qmoe_device.h")]
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def upload_weights(seed, shape, threads=16, chunk=32):
    import torch
    E, H, I = shape.E, shape.H, shape.I
    out = {
        "w13": torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
        "s13": torch.empty((E, 2 * I, H // 32), dtype=torch.int16, device="cuda"),
        "w2": torch.empty((E, H, I // 2), dtype=torch.uint8, device="cuda"),
        "s2": torch.empty((E, H, I // 32), dtype=torch.int16, device="cuda"),
    }
    with ThreadPoolExecutor(threads) as ex:
        for e0 in range(0, E, chunk):
            es = list(range(e0, min(E, e0 + chunk)))
            ws = list(ex.map(lambda e: synth.expert(seed, shape, e), es))
            for key in out:
                a = np.stack([w[key] for w in ws])
                if a.dtype == np.uint16:
                    a = a.view(np.int16)
                out[key][e0:e0 + len(es)].copy_(torch.from_numpy(a))
    shared = None
    if shape.shared:
        sh = synth.expert(seed, shape, "shared")
        shared = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda() for k, v in sh.items()}
    torch.cuda.synchronize()
    return out, shared


def bytes_per_expert(shape):
    H, I = shape.H, shape.I
    w13 = 2 * I * H // 2 + 2 * (2 * I * H // 32)
    w2 = H * I // 2 + 2 * (H * I // 32)
    return w13, w2


def source_hash():
    """Hash of the kernel sources: stored traffic counters apply only to the code they were taken on."""
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()[:16]


def stored_traffic(workload: str, M: int, path: str = COUNTERS):
    """HBM bytes per gate+up launch that the counter passes measured for this
    workload and M, or None when none were taken on the current kernel sources."""
    if not os.path.exists(path):
        return None
    try:
        c = json.load(open(path))
        if c.get("source_sha256_16") != source_hash():
            return None
        return c.get("gate_up_bytes_per_launch", {}).get(f"{workload}:M={M}")
    except (ValueError, AttributeError):
        return None


def cpu_baseline(shape, M, skew, budget_s=20.0):
    """The float64 oracle on the host: a full call when it fits the budget,
    else a sample of tokens; scaled to tokens/s."""
    from oracle import moe as oracle_moe
    inp = synth.inputs(0, shape, M, skew=skew)
    get = lambda e: synth.expert(0, shape, e)
    shared = synth.expert(0, shape, "shared") if shape.shared else None
    ntok = M if M <= 9 else 2
    tokens = np.arange(ntok)
    reps, dt = 0, 0.0
    while reps < 3 and (reps == 0 or dt < 10.0):  # at least ~10 s of work when one call is quick
        t0 = time.perf_counter()
        oracle_moe.forward(inp["x"], inp["logits"], shape.top_k, get, shape.I, shared=shared, tokens=tokens)
        dt += time.perf_counter() - t0
        reps += 1
    try:
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
    except ImportError:
        blas = []
    cores = max(blas) if blas else 1  # BLAS threads of the matmuls; the rest is one thread
    sample = (f"oracle (float64 numpy) on {ntok} of the {M} tokens of one call, routing for all {M}, "
              f"experts regenerated and decoded on the fly; {reps} run(s), {dt:.1f} s")
    return {"value": round(reps * ntok / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": sample}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: small calls (at most 64 tokens, well under a millisecond each)
    # get 50 warmup and 100 timed steps so the timed region runs at the
    # GPU's steady clocks; larger calls 5 and 20 (each step has its own
    # inputs, generated on the host)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--m", type=int, default=9)
    ap.add_argument("--workload", default="decode", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--also-m", default="1", help="comma list of extra M values timed the same way")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward captured into one HIP graph per step and replayed back to back")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device to device 5 times (reference reading for the HBM byte counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 1 GiB 5 times")
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested); "
              "the layer would shard by experts across GPUs, which is not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_mixture_experts_top_amd import Layer

    wl = synth.WORKLOADS[args.workload]
    shape = wl.shape
    Ms = [args.m] + [int(v) for v in args.also_m.split(",") if v.strip() and int(v) != args.m]
    max_rows = max(Ms)
    small = max_rows <= 64
    if args.steps is None:
        args.steps = 100 if small else 20
    if args.warmup is None:
        args.warmup = 50 if small else 5
    t0 = time.time()
    w, shared = upload_weights(0, shape)
    log(f"weights uploaded in {time.time() - t0:.1f} s")
    layer = Layer(E=shape.E, H=shape.H, I=shape.I, top_k=shape.top_k, max_rows=max_rows,
                  w13=w["w13"], s13=w["s13"], w2=w["w2"], s2=w["s2"], shared=shared)
    b13, b2 = bytes_per_expert(shape)
    stream = torch.cuda.current_stream()
    results = {}
    for M in Ms:
        n = args.warmup + args.steps
        xs, ls = [], []
        for s in range(n):
            inp = synth.inputs(0, shape, M, skew=wl.skew, logits_seed=1 + s)
            xs.append(torch.from_numpy(inp["x"].view(np.int16)).cuda().view(torch.bfloat16))
            ls.append(torch.from_numpy(inp["logits"]).cuda())
        out = torch.empty((M, shape.H), dtype=torch.bfloat16, device="cuda")
        layer.workspace(M)
        # experts touched by each step, from the layer's own routing
        touched = []
        for s in range(n):
            layer.route(xs[s], ls[s])
            c = layer.read_routing(M)["counts"]
            touched.append(int((c > 0).sum().item()) + (1 if shape.shared else 0))
        torch.cuda.synchronize()
        # ---- whole-layer throughput
        for s in range(args.warmup):
            layer.forward(xs[s], ls[s], out=out)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for s in range(args.warmup, n):
            layer.forward(xs[s], ls[s], out=out)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        # ---- per-kernel durations: the same four kernels, bracketed by events
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        for i, s in enumerate(range(args.warmup, n)):
            e = evs[i]
            e[0].record(stream)
            layer.route(xs[s], ls[s])
            e[1].record(stream)
            layer.gate_up(M)
            e[2].record(stream)
            layer.down(M)
            e[3].record(stream)
            layer.combine(M, out=out)
            e[4].record(stream)
        torch.cuda.synchronize()
        stage = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)] for i in range(args.steps)])
        # per-call distribution from the same bracketed loop (first to last event of each call)
        per_call_us = np.array([evs[i][0].elapsed_time(evs[i][4]) for i in range(args.steps)]) * 1e3
        # ---- optional: the same steps as captured graphs (one per step's inputs)
        graph = None
        if args.graph:
            outs = [torch.empty_like(out) for _ in range(n)]
            graphs = []
            torch.cuda.synchronize()
            for s in range(n):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    layer.forward(xs[s], ls[s], out=outs[s])
                graphs.append(g)
            for s in range(args.warmup):
                graphs[s].replay()
            torch.cuda.synchronize()
            gv0, gv1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gv0.record(stream)
            for s in range(args.warmup, n):
                graphs[s].replay()
            gv1.record(stream)
            torch.cuda.synchronize()
            eager_last = layer.forward(xs[n - 1], ls[n - 1])
            torch.cuda.synchronize()
            graph = {"us_per_call": gv0.elapsed_time(gv1) / args.steps * 1e3,
                     "matches_eager": bool(torch.equal(outs[n - 1].view(torch.int16), eager_last.view(torch.int16)))}
            del graphs, outs
        st_ms = stage.mean(axis=0)
        tt = np.array(touched[args.warmup:], dtype=np.float64)
        alg_bytes = tt * (b13 + b2) + M * shape.H * 2 + M * shape.E * 4 + M * shape.H * 2
        gu_bytes = tt * b13 + M * shape.H * 2
        dn_bytes = tt * b2 + M * shape.H * 2
        flops = 2.0 * (M * shape.top_k + (M if shape.shared else 0)) * 3 * shape.H * shape.I
        results[M] = {
            "us_per_call": ms * 1e3, "us_per_token": ms * 1e3 / M, "tokens_per_s": M / (ms * 1e-3),
            "experts_touched_mean": float(tt.mean()),
            "layer_GBps": float(alg_bytes.mean() / (ms * 1e-3) / 1e9),
            "layer_TFLOPs": flops / (ms * 1e-3) / 1e12,
            "stage_us": {"route": st_ms[0] * 1e3, "gate_up": st_ms[1] * 1e3, "down": st_ms[2] * 1e3,
                         "combine": st_ms[3] * 1e3},
            "gate_up_GBps": float(np.mean(gu_bytes / (stage[:, 1] * 1e-3)) / 1e9),
            "down_GBps": float(np.mean(dn_bytes / (stage[:, 2] * 1e-3)) / 1e9),
            "gate_up_TFLOPs": float(np.mean(2.0 * (M * shape.top_k + (M if shape.shared else 0)) * 2 * shape.H
                                            * shape.I / (stage[:, 1] * 1e-3)) / 1e12),
            "gate_up_bytes_per_launch": float(gu_bytes.mean()),
            "gate_up_us": float(st_ms[1] * 1e3),
            "bracketed_call_us_p10_p50_p90": [float(np.percentile(per_call_us, q)) for q in (10, 50, 90)],
        }
        if graph is not None:
            results[M]["graph_us_per_call"] = graph["us_per_call"]
            results[M]["graph_matches_eager"] = graph["matches_eager"]
        if graph is not None:
            log(f"M={M}: graph replay {graph['us_per_call']:.1f} us/call (matches eager: {graph['matches_eager']})")
        log(f"M={M}: {ms * 1e3:.1f} us/call, {results[M]['tokens_per_s']:.0f} tok/s, "
            f"{results[M]['layer_GBps']:.0f} GB/s layer, stages(us) "
            + ", ".join(f"{k}={v:.1f}" for k, v in results[M]["stage_us"].items()))
        del xs, ls

    M = args.m
    r = results[M]
    mfma_bound = r["gate_up_TFLOPs"] / MFMA_PEAK_TFLOPS > r["gate_up_GBps"] / HBM_PEAK_GBS
    traffic = stored_traffic(args.workload, M)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(r["gate_up_TFLOPs"], 2), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(r["gate_up_TFLOPs"] / MFMA_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(r["gate_up_GBps"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(r["gate_up_GBps"] / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic
    # both fractions, whichever binds (the plateau sits near the ridge)
    roof["hbm_frac"] = round(r["gate_up_GBps"] / HBM_PEAK_GBS, 4)
    roof["mfma_frac"] = round(r["gate_up_TFLOPs"] / MFMA_PEAK_TFLOPS, 4)
    roof["kernel"] = "gate_up (stacked gate+up grouped GEMM, SiLU*up epilogue)"
    roof["kernel_us"] = round(r["gate_up_us"], 2)
    roof["algorithmic_bytes_per_launch"] = round(r["gate_up_bytes_per_launch"])
    page = PAGE_MS_PER_CALL.get(M) if args.workload in ("decode", "transition", "plateau") else None
    line = {
        "metric": METRIC,
        "value": round(r["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["us_per_call"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(r["tokens_per_s"] / (M / (page * 1e-3)), 3) if page else None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} E={shape.E} H={shape.H} I={shape.I} top-{shape.top_k} "
                               f"int4-g32{' +shared' if shape.shared else ''} M={M}",
                   "E": shape.E, "H": shape.H, "I": shape.I, "top_k": shape.top_k, "M": M,
                   "group_size": 32, "shared_expert": shape.shared, "skew": wl.skew},
        "us_per_call": round(r["us_per_call"], 2),
        "us_per_token": round(r["us_per_token"], 3),
        "roofline": roof,
        "per_M": {str(m): {k: (round(v, 3) if isinstance(v, float) else
                               {kk: round(vv, 2) for kk, vv in v.items()} if isinstance(v, dict) else
                               [round(vv, 2) for vv in v] if isinstance(v, list) else v)
                           for k, v in results[m].items()} for m in Ms},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(shape, M, wl.skew)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
