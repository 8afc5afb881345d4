#!/usr/bin/env python3
"""Throughput of the fused MoE + multi-LoRA layer on one MI355X.

One step = one call of moe_lora_forward (route, align, LoRA shrink, gate_up GEMM with LoRA
expand and SiLU-and-mul, LoRA shrink, down GEMM with LoRA expand, combine) over one batch of
seeded synthetic input already resident in HBM. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode] [--fp8]

--fp8 runs the FP8 entry point (E4M3 expert weights with per-row scales, moe_lora_forward_fp8)
on any workload. --routed starts each step from router weights
(moe_lora_forward_routed: the router GEMM joins the step; the logits come from a seeded router
weight scaled to unit spread, so the workload's own logits, and fg's hot experts, are not used).
--workload sgmv measures the dense multi-LoRA entry point (moe_lora_sgmv) instead of the layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def algorithmic_work(w, seg_table, n_seg, topk_ids, fp8: bool = False):
    """Bytes and flops the method must move / compute for this routing (no padding, no
    intermediates): touched expert weights, touched (expert, adapter) LoRA weights, x,
    logits, adapter ids, y. Also the gate_up kernel's own share. With fp8 the expert weights
    are 1 byte each plus a 4-byte scale per weight row."""
    import numpy as np
    ids = topk_ids.cpu().numpy()
    seg = seg_table.cpu().numpy()[:n_seg]
    h, I, r, T, E, k = w.hidden, w.inter, w.rank, w.T, w.n_experts, w.topk
    n_exp = len(np.unique(ids))
    n_ea = int((seg[:, 1] >= 0).sum())  # (expert, adapter) segments that carry an adapter
    P = T * k
    pairs_with_adapter = int(seg[seg[:, 1] >= 0, 3].sum())
    wb = 1 if fp8 else 2  # bytes per expert weight
    sc = 4 if fp8 else 0   # scale bytes per weight row
    layer_bytes = (n_exp * (3 * h * I * wb + (2 * I + h) * sc) + n_ea * r * (2 * h + 3 * I) * 2
                   + 2 * T * h + 4 * T * E + 4 * T + 2 * T * h)
    layer_flops = 2 * P * 3 * h * I + 2 * pairs_with_adapter * r * (2 * h + 3 * I)
    gateup_bytes = (n_exp * 2 * I * (h * wb + sc) + n_ea * 2 * I * r * 2 + 2 * T * h + 2 * P * I
                    + 4 * pairs_with_adapter * r)
    gateup_flops = 2 * P * 2 * I * h + 2 * pairs_with_adapter * 2 * I * r
    return dict(n_experts_touched=n_exp, n_expert_adapter=n_ea, layer_bytes=layer_bytes,
                layer_flops=layer_flops, gateup_bytes=gateup_bytes, gateup_flops=gateup_flops)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lora_mixture_experts_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per gate_up launch from the committed rocprofv3 counter summary
    (profiles/traffic_gate_up_<workload>.txt: FETCH_SIZE and WRITE_SIZE scaled by a 1 GiB copy),
    or None when the summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line:
            key, val = line.split(":", 1)
            rec[key.strip()] = val.strip()
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu() -> dict:
    """CPU model and the threads this process may use (for the oracle baseline)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"model": model, "logical_cpus_available": avail}


def onbox_peaks(torch, ml, dev) -> dict:
    """The ceilings this box sustains, measured with the library's probes: a streaming read of
    4 GiB (HBM) and a loop of independent bf16 32x32x16 MFMAs on every SIMD (two wavefronts
    each); best of 5 launches after one warm-up, timed with events on the launch stream."""
    src = torch.empty(4 << 30, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty(ml.PROBE_READ_SINK, dtype=torch.int32, device=dev)
    fsink = torch.empty(512 * 256, dtype=torch.float32, device=dev)

    def best(fn, n=5):
        times = []
        fn()
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        return min(times)

    t_read = best(lambda: ml.probe_read(src, sink))
    read_bytes = src.numel() + sink.numel() * 4
    flops = [0]

    def mf():
        flops[0] = ml.probe_mfma(20000, 512, fsink)

    t_mfma = best(mf)
    del src
    torch.cuda.empty_cache()
    return {"hbm_read_GBs": read_bytes / t_read / 1e9, "mfma_bf16_TFLOPs": flops[0] / t_mfma / 1e12,
            "how": "moe_lora_probe_read over 4 GiB; moe_lora_probe_mfma, 512 workgroups x 4 "
                   "wavefronts x 20000 x 8 MFMAs 32x32x16 bf16; best of 5 launches"}


def call_stats(ms: list) -> dict:
    ms = sorted(ms)

    def q(f):
        i = f * (len(ms) - 1)
        lo = int(math.floor(i))
        hi = min(lo + 1, len(ms) - 1)
        return ms[lo] + (ms[hi] - ms[lo]) * (i - lo)

    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "n": len(ms)}


def cpu_baseline(w, inp, n_tokens: int, min_seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload (host copies made
    before timing), run over the sample repeatedly until at least min_seconds have passed."""
    import numpy as np
    import torch
    import oracle
    toks = np.linspace(0, w.T - 1, num=min(n_tokens, w.T)).round().astype(np.int32)
    toks = np.unique(toks)
    tok_t = torch.from_numpy(toks.astype(np.int64)).to(inp["x"].device)
    ad = inp["adapter_ids"].index_select(0, tok_t).cpu().numpy()
    used = sorted({int(a) for a in ad if a >= 0}) or [0]
    remap = {a: i for i, a in enumerate(used)}
    used_t = torch.tensor(used, dtype=torch.int64, device=inp["x"].device)
    host = {"x": inp["x"].index_select(0, tok_t).cpu(), "logits": inp["logits"].index_select(0, tok_t).cpu(),
            "adapter_ids": np.array([remap.get(int(a), -1) for a in ad], np.int32),
            "W1": inp["W1"].cpu(), "W2": inp["W2"].cpu()}
    for n in ("W1_scale", "W2_scale"):
        if n in inp:
            host[n] = inp[n].cpu()
    for n in ("A1", "B1", "A2", "B2"):
        host[n] = inp[n].index_select(0, used_t).cpu()
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(host, w.topk)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": passes * len(toks) / dt, "unit": "tokens/s",
            "cores": min(oracle.num_threads(), len(toks)), "kind": "oracle",
            "sample": f"{passes} passes over {len(toks)} of {w.T} tokens of the {w.name} batch, fp64 C "
                      f"oracle with OpenMP over tokens, inputs already in host memory; {dt:.1f} s wall",
            "host": host_cpu()}


# dense multi-LoRA: a serving batch of 256 tokens on a 4096 x 4096 projection, 64 adapters of
# rank 16, one adapter per request of 4 tokens (uniform over the adapters)
SGMV = dict(T=256, K=4096, N=4096, nA=64, r=16, run=4)


def run_sgmv(args, torch, ml, dev):
    """moe_lora_sgmv over seeded inputs in HBM: value = tokens/s; roofline = the call's
    algorithmic bytes (touched A and B slabs, x, y read and written) over its time."""
    import numpy as np
    c = SGMV
    g = torch.Generator().manual_seed(args.seed)
    T, K, N, nA, r = c["T"], c["K"], c["N"], c["nA"], c["r"]
    x = (torch.randn(T, K, generator=g) * 0.02).to(torch.bfloat16)
    A = (torch.randn(nA, r, K, generator=g) * 0.02).to(torch.bfloat16)
    B = (torch.randn(nA, N, r, generator=g) * 0.02).to(torch.bfloat16)
    ad = torch.randint(0, nA, (T // c["run"] + 1,), generator=g, dtype=torch.int32).repeat_interleave(c["run"])[:T]
    y = torch.zeros(T, N, dtype=torch.bfloat16)
    xd, Ad, Bd, add, yd = (t.to(dev) for t in (x, A, B, ad, y))
    d = ml.SgmvDims(T, K, N, nA, r)
    import ctypes
    ws = torch.empty(int(ml.lib().moe_lora_sgmv_workspace_size(ctypes.byref(d))), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        ml.sgmv(xd, Ad, Bd, add, yd, workspace=ws)
    torch.cuda.synchronize()
    # the timed region: K back-to-back calls (value); then K more calls, each between two events
    # on its stream, for the per-call GPU time of its three launches (median and spread; the
    # roofline uses the median)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ml.sgmv(xd, Ad, Bd, add, yd, workspace=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        ml.sgmv(xd, Ad, Bd, add, yd, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in evs]
    st = call_stats(call_ms)
    n_ad = len(np.unique(ad.numpy()))
    nbytes = n_ad * r * (K + N) * 2 + T * K * 2 + 2 * T * N * 2 + 4 * T
    per_call = st["median"] * 1e-3
    ach = nbytes / per_call / 1e9
    out = {
        "metric": "tokens/s of the dense multi-LoRA (SGMV) add",
        "value": T * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True,
        "call_ms": st,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "sgmv", "T": T, "in_features": K, "out_features": N,
                   "n_adapters": nA, "rank": r, "tokens_per_adapter_run": c["run"], "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "whole call (3 launches), median of per-call event times"},
    }
    if not args.no_cpu_baseline:
        import oracle
        toks = np.arange(0, T, max(1, T // 32))
        xs, ys, ads = x[toks], y[toks].float().to(torch.bfloat16), ad[toks]
        passes, t1 = 0, time.perf_counter()
        while True:
            oracle.sgmv(xs, A, B, ys, ads)
            passes += 1
            dt = time.perf_counter() - t1
            if dt >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {"value": passes * len(toks) / dt, "unit": "tokens/s",
                               "cores": min(oracle.num_threads(), len(toks)), "kind": "oracle",
                               "sample": f"{passes} passes over {len(toks)} of {T} tokens, fp64 C oracle; {dt:.1f} s wall",
                               "host": host_cpu()}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "fg", "stress_distinct", "stress_same", "tiny", "sgmv"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=64, help="oracle sample size (tokens)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle over its sample for at least this long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="E4M3 expert weights with per-row scales (moe_lora_forward_fp8)")
    ap.add_argument("--routed", action="store_true",
                    help="start from router weights: moe_lora_forward_routed (router GEMM in the step)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the on-box HBM-read and MFMA-loop probes")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a device-to-device copy of this size first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X; multi-GPU "
              "(expert-parallel) runs are not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    import lora_mixture_experts_amd as ml
    from synth import configs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.workload == "sgmv":
        run_sgmv(args, torch, ml, dev)
        return
    w = configs.WORKLOADS[args.workload]

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.fp8 and args.routed:
        print("--routed covers the bf16 entry point", file=sys.stderr)
        sys.exit(2)
    inp = (configs.make_inputs_fp8 if args.fp8 else configs.make_inputs)(w, args.seed, device=dev)
    Wr = None
    if args.routed:
        # router weight whose logits x W_router^T have about unit spread (like the workload's)
        g = torch.Generator().manual_seed(args.seed + 7)
        sx = float(inp["x"].float().std())
        Wr = (torch.randn(w.n_experts, w.hidden, generator=g) / (sx * math.sqrt(w.hidden))).to(
            torch.bfloat16).to(dev)
        inp["logits"] = ml.router_logits(inp["x"], Wr)  # what the routed entry computes
    d = ml.Dims(w.T, w.hidden, w.inter, w.n_experts, w.n_adapters, w.rank)
    ws = ml.new_workspace(d, w.topk, dev)
    y = torch.empty((w.T, w.hidden), dtype=torch.bfloat16, device=dev)

    ra = ml.route_align(inp["logits"], inp["adapter_ids"], w.topk, d, 1, 1, workspace=ws)
    work = algorithmic_work(w, ra["seg_table"], int(ra["n_seg"].item()), ra["topk_ids"], args.fp8)
    if args.routed:  # the router weight read and the router GEMM
        work["layer_bytes"] += 2 * w.n_experts * w.hidden
        work["layer_flops"] += 2 * w.T * w.hidden * w.n_experts
    del ra

    keys = ("W1", "W2", "A1", "B1", "A2", "B2", "adapter_ids")

    def step(events=None):
        if args.routed and events is None:
            ml.forward_routed(inp["x"], Wr, *[inp[k] for k in keys], w.topk, y=y, workspace=ws)
        elif args.routed:
            # the routed entry's kernels, with the router GEMM and every stage boundary timed
            events[-1][0].record()
            ml.router_logits(inp["x"], Wr, out=inp["logits"])
            events[-1][1].record()
            ml.forward(inp["x"], inp["logits"], *[inp[k] for k in keys], w.topk, y=y, workspace=ws,
                       stage_events=events[:-1])
        elif args.fp8:
            ml.forward_fp8(inp["x"], inp["logits"], inp["W1"], inp["W1_scale"], inp["W2"],
                           inp["W2_scale"], inp["A1"], inp["B1"], inp["A2"], inp["B2"],
                           inp["adapter_ids"], w.topk, y=y, workspace=ws, stage_events=events)
        else:
            ml.forward(inp["x"], inp["logits"], inp["W1"], inp["W2"], inp["A1"], inp["B1"], inp["A2"],
                       inp["B2"], inp["adapter_ids"], w.topk, y=y, workspace=ws, stage_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole-layer calls. Only the two events around the gate_up launch are
    # recorded (every event record adds a gap between launches); the other stages are timed in
    # a separate pass after the timed region.
    K = args.steps
    GU = ml.STAGES.index("gate_up")
    if args.routed:
        # the routed entry records no stage events: gate_up and the router GEMM are timed in the
        # breakdown pass below, over the same kernels
        call_events = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        for ev in call_events:
            ev.record()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            call_events[i].record()
            step()
        call_events[K].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        call_ms = [call_events[i].elapsed_time(call_events[i + 1]) for i in range(K)]
    else:
        gu_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        # one event at the start of every call and one after the last: per-call GPU times
        call_events = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        for ev in [e for evs in gu_events for e in evs] + call_events:
            ev.record()  # create the HIP events outside the timed region
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            evs = [None] * (ml.N_STAGES + 1)
            evs[0] = call_events[i]
            evs[GU], evs[GU + 1] = gu_events[i]
            step(evs)
        call_events[K].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        gu_ms = statistics.fmean(a.elapsed_time(b) for a, b in gu_events)
        call_ms = [call_events[i].elapsed_time(call_events[i + 1]) for i in range(K)]

    # stage breakdown (diagnostics): a few more calls with every boundary recorded
    NB = min(K, 5) if not args.routed else K
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(ml.N_STAGES + 1)] for _ in range(NB)]
    if args.routed:
        for evs in events:
            evs.append([torch.cuda.Event(enable_timing=True) for _ in range(2)])
    for i in range(NB):
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = {name: [] for name in ml.STAGES}
    if args.routed:
        stage_ms = {"router": [evs[-1][0].elapsed_time(evs[-1][1]) for evs in events], **stage_ms}
    for evs in events:
        for s, name in enumerate(ml.STAGES):
            stage_ms[name].append(evs[s].elapsed_time(evs[s + 1]))
    stage_avg = {k: statistics.fmean(v) for k, v in stage_ms.items()}
    if args.routed:
        gu_ms = stage_avg["gate_up"]

    ms_per_step = elapsed * 1e3 / K
    value = w.T * K / elapsed
    prefill_like = args.workload == "prefill"
    gu_s = gu_ms * 1e-3
    if prefill_like:
        achieved = work["gateup_flops"] / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS}
    else:
        achieved = work["gateup_bytes"] / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    # the library takes the LDS-tiled GEMM above 24 rows per expert on average
    tiled = w.T * w.topk > 24 * w.n_experts
    roof["kernel"] = ("tiled_gemm_kernel" if tiled else "skinny_gemm_kernel") + " (gate_up)"
    roof["traffic"] = measured_traffic(args.workload + ("_fp8" if args.fp8 else "")
                                       + ("_routed" if args.routed else ""))

    layer_s = elapsed / K
    cs = call_stats(call_ms)
    onbox = None if args.no_probes else onbox_peaks(torch, ml, dev)
    if onbox:
        roof["frac_onbox"] = roof["achieved"] / (onbox["mfma_bf16_TFLOPs"] if prefill_like
                                                 else onbox["hbm_read_GBs"])
    out = {
        "metric": "tokens/s of fused MoE-LoRA layer",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 expert weights, bf16 activations" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "hidden": w.hidden, "inter": w.inter,
                   "n_experts": w.n_experts, "topk": w.topk, "n_adapters": w.n_adapters,
                   "rank": w.rank, "adapters": w.adapters, "seed": args.seed,
                   "expert_weights": "e4m3 + per-row fp32 scale" if args.fp8 else "bf16",
                   "logits": "x W_router^T (routed entry)" if args.routed else "given"},
        "roofline": roof,
        "call_ms": cs,
        "layer": {"bytes": work["layer_bytes"], "flops": work["layer_flops"],
                  "ms": layer_s * 1e3,
                  "hbm_frac": work["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBS,
                  "mfma_frac": work["layer_flops"] / layer_s / 1e12 / BF16_PEAK_TFLOPS},
        "stages_ms": {k: round(v, 4) for k, v in stage_avg.items()},
    }
    if onbox:
        out["onbox_peaks"] = onbox
        out["layer"]["hbm_frac_onbox"] = work["layer_bytes"] / layer_s / 1e9 / onbox["hbm_read_GBs"]
        out["layer"]["mfma_frac_onbox"] = work["layer_flops"] / layer_s / 1e12 / onbox["mfma_bf16_TFLOPs"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_tokens, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
