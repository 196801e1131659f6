"""Benchmark of the DeepSeekMoE layer forward on one MI355X.

One step = one whole layer pass through the C ABI on synthetic seeded inputs
already resident in HBM: moe_route -> moe_permute -> moe_expert_ffn (bf16: the
up and down projections in one fused launch) -> moe_combine ->
moe_balance_stats.  Prints ONE JSON line.

Default workload: the largest single-GPU prefill layer, a 145B-style layer
(T=8192 tokens, d=4096, 4 shared + 128 routed experts of width 1024, top-12,
bf16).  The granularity-equivalence pair (fine-grained: 64 experts of width
512, top-8; coarse GShard-style: 16 experts of width 2048, top-2; T=4096,
d=1280, same weights) is timed alongside under "pair" (--no-pair skips it).
Other workloads: --config.  --accumulate runs moe_expert_ffn in its
accumulating mode (gate-weighted sum inside the down projection, no y_routed).

"layer_forward" times the same pass as one moe_layer_forward call (decode
batches: four kernels instead of seven; other batches: the five calls' kernels).

Timing: W warm-up steps, then K steps between two device synchronisations
(value, ms_per_step); then a separate loop of max(K, 50) steps (200 for
decode batches) with an event pair around each step gives the median and the
minimum step time.  The dominant kernel's time is the mean of event pairs
around every moe_expert_ffn call of the K timed steps.

Extra modes (used to produce the committed profile summaries):
  --copy-probe       also run a plain device copy of known size (counter calibration)
  --backward         time the backward pass instead (moe_combine_backward ->
                     moe_expert_ffn_backward -> moe_route_backward after one forward);
                     prints its own JSON line
  --ingest-pmc DIR   read rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs under DIR
                     and write profiles/traffic_<kernel>_<workload>.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + active TFLOP/s (% MFMA/HBM peak) on 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
# the source of the dominant kernel: a traffic record measured on other sources is not reported
KERNEL_SOURCES = ["fine_grained_mixture_moe_amd/csrc/expert_ffn.hip"]
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def ffn_algorithmic(wl, counts) -> dict:
    """Algorithmic work of one moe_expert_ffn call (both projections of every expert).

    Per (token, expert) pair: 6*d*w FLOPs (gate and up: 2 x 2*d*w, down: 2*d*w).
    Bytes: W1, W3 and W2 of every touched expert (all shared + routed experts with
    tokens), the token rows read once and the expert sum y written once (fp32).
    The SwiGLU activations and the per-pair rows y_routed are intermediates of an
    implementation (the gather mode writes y_routed, the accumulating mode does
    not): their HBM traffic shows in the measured FETCH/WRITE counters, and is
    not part of the algorithmic minimum.
    """
    es = 2 if wl.dtype == "bf16" else 4
    pairs = wl.T * (wl.top_k + wl.n_shared)
    flops = 6.0 * wl.d * wl.inter * pairs
    touched = wl.n_shared + int((counts > 0).sum())
    byts = 3.0 * wl.inter * wl.d * es * touched + wl.T * wl.d * es + wl.T * wl.d * 4
    return dict(flops=flops, bytes=byts, pairs=pairs, touched=touched)


def layer_bytes(wl, counts) -> float:
    """Algorithmic bytes of one layer pass: touched expert weights, x in, h out, centroids, routing table."""
    es = 2 if wl.dtype == "bf16" else 4
    touched = wl.n_shared + int((counts > 0).sum())
    return (3.0 * wl.inter * wl.d * es * touched + 2.0 * wl.T * wl.d * es + wl.n_routed * wl.d * 4
            + wl.T * wl.top_k * 8)


def load_traffic(kernel_tag: str, workload: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        log(f"[bench] {path} was measured on other kernel sources: traffic reported as null")
        return None
    return rec


def host_info() -> dict:
    """CPU model and core counts of the host the oracle runs on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def _oracle_args(inp):
    wl = inp.wl
    sh, ro = inp.shared, inp.routed
    return (inp.x.f32, inp.centroids, inp.bias, wl.top_k, max(wl.groups, 1), sh(inp.w1).f32, sh(inp.w3).f32,
            sh(inp.w2).f32, ro(inp.w1).f32, ro(inp.w3).f32, ro(inp.w2).f32)


def cpu_baseline(inp, budget_s: float = 15.0) -> dict:
    """The oracle (plain C, fp64 FFN, OpenMP over tokens) on a bounded sample of the workload,
    plus the whole tiny c1 layer on one thread."""
    from oracle import oracle as O
    from fine_grained_mixture_moe_amd import workloads as W
    wl = inp.wl
    args = _oracle_args(inp)
    n0 = min(wl.T, 64)
    t0 = time.perf_counter()
    O.forward(n0, *args)
    dt0 = time.perf_counter() - t0
    n = int(min(wl.T, max(n0, n0 * budget_s / max(dt0, 1e-6))))
    n = max(n0, n - n % 64) if n >= 64 else n
    t0 = time.perf_counter()
    O.forward(n, *args)
    dt = time.perf_counter() - t0
    threads = O.num_threads()
    out = {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"first {n} of {wl.T} tokens of the same workload, whole layer pass "
                     f"(route, group, fp64 expert FFNs, combine, stats); {dt:.1f} s on {threads} OpenMP threads",
           "tflops": wl.flops() * n / wl.T / dt / 1e12, "threads": threads}
    out.update(host_info())
    # the whole tiny fp32 layer (T=512, d=256, 1+63 experts, top-7, width 128) on one thread
    c1 = W.make_inputs(W.WORKLOADS["c1"])
    O.set_num_threads(1)
    try:
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            O.forward(c1.wl.T, *_oracle_args(c1))
            times.append(time.perf_counter() - t0)
    finally:
        O.set_num_threads(threads)
    t1 = sorted(times)[1]
    out["c1_one_thread"] = {"tokens_per_s": round(c1.wl.T / t1, 1), "seconds": round(t1, 4),
                            "runs": "median of 3", "threads": 1}
    return out


def device_info() -> dict:
    """The GPU the line was measured on (the peaks above are MI355X's published ones)."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "cus": pr.multi_processor_count,
            "hbm_gib": round(pr.total_memory / (1 << 30), 1)}


def run(args) -> dict:
    import numpy as np
    import torch
    from fine_grained_mixture_moe_amd import workloads as W
    from fine_grained_mixture_moe_amd.layer import DeviceLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    name = args.config
    t_gen = time.perf_counter()
    coarse = None
    if name in ("c2b", "c2a"):
        coarse = W.make_c2_coarse()
        inp = coarse if name == "c2a" else W.make_c2_fine(independent_centroids=True, coarse=coarse)
    else:
        inp = W.make_inputs(W.WORKLOADS[name])
    wl = inp.wl
    log(f"[bench] {name}: {wl.description} (inputs in {time.perf_counter() - t_gen:.1f}s)")
    dl = DeviceLayer(inp, device="cuda:0", accumulate=args.accumulate)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        dl.route()
        dl.permute()
        if ev is not None:
            ev[0].record(stream)
        dl.expert_ffn()
        if ev is not None:
            ev[1].record(stream)
        dl.combine()
        dl.balance_stats()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ffn_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ms = elapsed * 1e3 / args.steps
    counts = dl.counts.cpu().numpy()[:wl.n_routed]
    dl.check_status()     # a stalled wait inside the fused launch would have poisoned the outputs

    # per-step distribution: an event pair around every step
    decode = wl.T * max(wl.top_k, 1) <= 64 * max(wl.n_routed, 1)
    reps = max(args.steps, 200 if decode else 50)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in sev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in sev)
    step_stats = {"reps": reps, "median_ms": round(per[len(per) // 2], 4), "min_ms": round(per[0], 4),
                  "max_ms": round(per[-1], 4)}

    # per-stage breakdown (separate, untimed-for-value loop)
    stages = ["route", "permute", "expert_ffn", "combine", "balance_stats"]
    n_b = min(args.steps, 10)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(n_b)]
    for i in range(n_b):
        marks[i][0].record(stream)
        for j, s in enumerate(stages):
            getattr(dl, s)()
            marks[i][j + 1].record(stream)
    torch.cuda.synchronize()
    # median per stage: a late host enqueue of one pass shows up as idle time before its first kernel
    breakdown = {s: round(sorted(m[j].elapsed_time(m[j + 1]) for m in marks)[n_b // 2], 4)
                 for j, s in enumerate(stages)}

    # the same pass as one moe_layer_forward call (decode batches: four kernels instead of seven)
    lf = None
    if wl.n_routed and not dl.accumulate:
        for _ in range(3):
            dl.layer_forward()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dl.layer_forward()
        torch.cuda.synchronize()
        lf_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in lev:
            a.record(stream)
            dl.layer_forward()
            b.record(stream)
        torch.cuda.synchronize()
        lper = sorted(a.elapsed_time(b) for a, b in lev)
        dl.check_status()
        lf = {"ms_per_step": round(lf_ms, 4), "median_ms": round(lper[len(lper) // 2], 4),
              "min_ms": round(lper[0], 4), "tokens_per_s": round(wl.T / (lf_ms * 1e-3), 1),
              "layer_hbm_gbs": round(layer_bytes(wl, counts) / (lf_ms * 1e-3) / 1e9, 1)}

    if args.copy_probe:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # an elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 3 x {COPY_BYTES} bytes")

    ffn = ffn_algorithmic(wl, counts)
    tflops = wl.flops() / (ms * 1e-3) / 1e12
    ai = ffn["flops"] / ffn["bytes"]
    mfma_peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    ridge = mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        achieved = ffn["flops"] / (ffn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(achieved / mfma_peak, 4)}
    else:
        achieved = ffn["bytes"] / (ffn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    tr = load_traffic("ffn", name)
    roof["traffic"] = None if tr is None else tr["bytes_per_launch"]
    # the kernel the launcher picks (template arguments: token-tile rows, weight-load cache
    # policy (2: nt), accumulating down projection); the events bracket the whole
    # moe_expert_ffn call: the fused launch plus the small preparation kernel before it
    from fine_grained_mixture_moe_amd import moe as M
    roof["kernel"] = M.moe_expert_ffn_kernel(dl.prob, dl.accumulate)
    roof["kernel_ms"] = round(ffn_ms, 4)
    roof["kernel_ms_includes"] = "ffn_prep_kernel + " + roof["kernel"]
    roof["algorithmic"] = {"flops": ffn["flops"], "bytes": ffn["bytes"], "pairs": ffn["pairs"],
                           "touched_experts": ffn["touched"]}

    out = {
        "metric": METRIC,
        "value": round(wl.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{name}: {wl.description}", "T": wl.T, "d": wl.d, "n_shared": wl.n_shared,
                   "n_routed": wl.n_routed, "top_k": wl.top_k, "inter": wl.inter, "parallelism": "none (1 GPU)",
                   "expert_ffn_mode": "accumulating" if dl.accumulate else "gather"},
        "step_ms": step_stats,
        "active_tflops": round(tflops, 2),
        "active_mfma_frac": round(tflops / mfma_peak, 4),
        "layer_hbm_gbs": round(layer_bytes(wl, counts) / (ms * 1e-3) / 1e9, 1),
        "stage_ms": breakdown,
        "layer_forward": lf,
        "roofline": roof,
        "device": device_info(),
    }
    if not args.no_pair:
        out["pair"] = time_pair(args, ms if name == "c2b" else None)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    return out


def time_pair(args, ms_b=None) -> dict:
    """The granularity-equivalence pair: fine-grained (64 x 512, top-8) and coarse (16 x 2048, top-2)
    layers on the same weights and tokens, equal active FLOPs; whole-layer step times."""
    import torch
    from fine_grained_mixture_moe_amd import workloads as W
    from fine_grained_mixture_moe_amd.layer import DeviceLayer
    coarse = W.make_c2_coarse()
    res = {}
    for key, inp in (("c2a", coarse), ("c2b", W.make_c2_fine(independent_centroids=True, coarse=coarse))):
        if key == "c2b" and ms_b is not None:
            res["c2b_ms_per_step"] = round(ms_b, 4)
            continue
        dl = DeviceLayer(inp, device="cuda:0", accumulate=args.accumulate)
        for _ in range(args.warmup):
            dl.forward()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = max(args.steps, 20)
        for _ in range(n):
            dl.forward()
        torch.cuda.synchronize()
        res[f"{key}_ms_per_step"] = round((time.perf_counter() - t0) * 1e3 / n, 4)
        del dl
    res["fine_over_coarse_time"] = round(res["c2b_ms_per_step"] / res["c2a_ms_per_step"], 3)
    return res


def run_backward(args) -> dict:
    """Backward pass of the layer: upstream gradient dh (seeded), alpha1 = alpha2 = 0.01."""
    import numpy as np
    import torch
    from fine_grained_mixture_moe_amd import workloads as W
    from fine_grained_mixture_moe_amd.layer import DeviceLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    name = args.config
    inp = W.make_c2_fine(independent_centroids=True) if name == "c2b" else (
        W.make_c2_coarse() if name == "c2a" else W.make_inputs(W.WORKLOADS[name]))
    wl = inp.wl
    dl = DeviceLayer(inp, device="cuda:0", want_probs=True)
    dl.forward()
    rng = np.random.default_rng(1234)
    dh = rng.standard_normal((wl.T, wl.d)).astype(np.float32)
    stream = torch.cuda.current_stream()
    dl.backward(dh, 0.01, 0.01)      # allocates the gradient buffers
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        dl.backward(dh, 0.01, 0.01)
    torch.cuda.synchronize()
    # time the three calls without the host-side dh upload: reuse the uploaded dh
    import fine_grained_mixture_moe_amd.moe as M
    p = dl.prob

    def calls(marks=None):
        if marks:
            marks[0].record(stream)
        if p.n_routed:
            M.moe_combine_backward(p, dl.dh, dl.y_routed, dl.gate, dl.slot_of, dl.dy_routed, dl.dgate)
        if marks:
            marks[1].record(stream)
        M.moe_expert_ffn_backward(p, dl.x, dl.offsets, dl.sorted_token, dl.slot_of, dl.w1_r, dl.w3_r, dl.w2_r,
                                  dl.w1_s, dl.w3_s, dl.w2_s, dl.dh, dl.dy_routed, dl.dx_ffn, dl.dw1_r, dl.dw3_r,
                                  dl.dw2_r, dl.dw1_s, dl.dw3_s, dl.dw2_s, dl.bws, dl.bws_bytes)
        if marks:
            marks[2].record(stream)
        if p.n_routed:
            M.moe_route_backward(p, max(dl.groups, 1), 0.01, 0.01, dl.x, dl.centroids, dl.probs, dl.idx, dl.dgate,
                                 dl.f, dl.f_dev, dl.dh, dl.dx_ffn, dl.dx, dl.dcent, dl.dbias, dl.bws, dl.bws_bytes)
        if marks:
            marks[3].record(stream)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        calls()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(min(args.steps, 10))]
    for m in marks:
        calls(m)
    torch.cuda.synchronize()
    stages = {k: round(sorted(m[j].elapsed_time(m[j + 1]) for m in marks)[len(marks) // 2], 4)
              for j, k in enumerate(["combine_backward", "expert_ffn_backward", "route_backward"])}
    pairs = wl.T * (wl.top_k + wl.n_shared)
    ffn_flops = 16.0 * wl.d * wl.inter * pairs
    router_flops = 4.0 * wl.T * wl.d * wl.n_routed
    mfma_peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    ffn_ms = stages["expert_ffn_backward"]
    return {
        "metric": "MoE-layer backward tokens/s (dh -> dx, dW, dcentroids) on 1 MI355X",
        "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": wl.dtype,
        "data": "synthetic", "config": {"workload": f"{name}: {wl.description}", "alpha1": 0.01, "alpha2": 0.01},
        "stage_ms": stages,
        "expert_ffn_backward": {"flops": ffn_flops, "tflops": round(ffn_flops / (ffn_ms * 1e-3) / 1e12, 2),
                                "frac_of_mfma_peak": round(ffn_flops / (ffn_ms * 1e-3) / 1e12 / mfma_peak, 4)},
        "active_tflops": round((ffn_flops + router_flops) / (ms * 1e-3) / 1e12, 2),
    }


def ingest_pmc(pmc_dir: str, workload: str) -> None:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the fused expert-FFN kernel, scaled by the copy
    probe's readings."""
    rows = []
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    per = {}
    for r in rows:
        kname = r.get("Kernel_Name", "")
        cname = r.get("Counter_Name", "")
        if "grouped_ffn_fused_kernel" in kname:
            key = "ffn"
        elif "elementwise" in kname.lower():
            key = "copy"
        else:
            continue
        per.setdefault((key, cname), []).append(float(r["Counter_Value"]))
    rec = {"workload": workload, "source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = per.get(("copy", cname))
        k = per.get(("ffn", cname))
        if not cp or not k:
            continue
        # copy reads COPY_BYTES and writes COPY_BYTES: bytes per counter unit
        copy_kib = max(cp)
        scale = COPY_BYTES / copy_kib
        rec[cname] = {"kib_per_dispatch": sum(k) / len(k), "dispatches": len(k), "copy_kib": copy_kib,
                      "bytes_per_unit": scale, "bytes": sum(k) / len(k) * scale}
    if "FETCH_SIZE" in rec and "WRITE_SIZE" in rec:
        rec["bytes_per_launch"] = rec["FETCH_SIZE"]["bytes"] + rec["WRITE_SIZE"]["bytes"]
    out = os.path.join(ROOT, "profiles", f"traffic_ffn_{workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def summarize_trace(trace_dir: str, command: str) -> None:
    """Text summary of a rocprofv3 --kernel-trace --stats run (kernel_stats.csv)."""
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(paths[0])))
    print(f"# rocprofv3 kernel statistics")
    print(f"# command: {command}")
    print(f"# {'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_%':>8s}")
    for r in rows:
        name = r["Name"].replace("moe::(anonymous namespace)::", "").replace("void ", "")
        name = name.split("(")[0][:70]
        print(f"  {name:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
              f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c5b", help="c1 c2a c2b c3 c4 c5a c5b c5c")
    ap.add_argument("--accumulate", action="store_true",
                    help="accumulating expert FFN (gate-weighted sum inside the down projection)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-pair", action="store_true", help="skip timing the c2a/c2b granularity pair")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--backward", action="store_true", help="time the backward pass (own JSON line)")
    ap.add_argument("--ingest-pmc", default=None)
    ap.add_argument("--summarize-trace", default=None, help="rocprofv3 output dir to summarize")
    ap.add_argument("--trace-command", default="", help="command that produced --summarize-trace")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc, args.config)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.trace_command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this layer pass has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    out = run_backward(args) if args.backward else run(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
