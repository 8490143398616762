"""Benchmark of the fused attention forward pass on one MI355X.

One step is one call of the whole forward pass (score, mask, online
softmax, weighted sum of V, output) over one batch of synthetic inputs that
already sit in device memory. Default workload: GQA bf16, B=2, Hq=32, Hkv=8,
S=4096, D=128, causal. Throughput is attention TFLOP/s with the causal
FLOPs counted as half (4 B Hq Sq Skv D / 2), next to the MI355X dense bf16
matrix-core peak, and next to the fp64 CPU oracle timed on a bounded sample of
the same workload on this host's cores.

Before timing: W warmup steps, then untimed steps for at least SETTLE_S seconds,
so the GPU runs at its sustained clock (after idle it needs tens of ms of load).

Prints ONE JSON line on stdout. ``--sweep-out FILE`` additionally writes one
JSON line per named workload (sequence and batch sweeps included) to FILE.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA peak at S=4096 causal GQA bf16"
# MI355X published dense peaks (TFLOP/s) by arithmetic type of the products.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "f32": 157.3}
PEAK_KIND = {"bf16": "mfma", "f16": "mfma", "e4m3": "mfma", "f32": "alu"}
PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E
N_BUFFER_SETS = 4   # rotating input sets, so one call's inputs are not cache-warm from the last
SETTLE_S = 0.25     # seconds of untimed steps after the warmup steps, before timing


# The sources a workload's kernels are built and launched from: a committed
# traffic figure stays valid while these are unchanged.
KERNEL_SOURCES = {
    "fwd": ["attn_fwd_mfma.hip", "attn_combine.hip", "mfma_common.h", "kernel_common.h", "attn_api.cpp"],
    "bwd": ["attn_bwd.hip", "attn_fwd_mfma.hip", "mfma_common.h", "kernel_common.h", "attn_api.cpp"],
}


def kernel_source_hash(direction="fwd"):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_dot_product_09_amd", "csrc")
    for f in KERNEL_SOURCES[direction]:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(w):
    """HBM bytes per call from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters, or None if there are none for this workload or its kernel
    sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(w.name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_hash") != kernel_source_hash(w.direction):
        return None
    return rec.get("traffic_bytes")


def describe(w):
    """The workload's shape in words, e.g. "bf16 GQA B=2 Hq=32 Hkv=8 S=4096 D=128 causal"."""
    kind = "MHA" if w.Hq == w.Hkv else ("MQA" if w.Hkv == 1 else "GQA")
    heads = f"H={w.Hq}" if w.Hq == w.Hkv else f"Hq={w.Hq} Hkv={w.Hkv}"
    seq = f"S={w.Sq}" if w.Sq == w.Skv else f"Sq={w.Sq} Skv={w.Skv}"
    mask = {False: "", True: " causal", "bottom_right": " bottom-right causal"}[w.causal]
    extra = []
    if w.layout != "bshd":
        extra.append(f"{w.layout.upper()} storage, strided entry point")
    if w.n_split is not None:
        extra.append("split keys")
    if w.scaling == "delayed":
        extra.append("delayed-scaling step: casts + attention + update")
    tail = f" ({', '.join(extra)})" if extra else ""
    return f"{w.dtype} {kind} B={w.B} {heads} {seq} D={w.D}{mask}{tail}"


def metric_name(w):
    """The headline workload carries the headline metric; every other line
    names its own workload."""
    from scaled_dot_product_09_amd import workload
    if w.name == workload.HEADLINE:
        return METRIC
    if w.direction == "bwd":
        return (f"attention bwd TFLOP/s (2.5x the forward's FLOPs: the five products of the gradients), "
                f"{describe(w)}")
    return f"attention fwd TFLOP/s and % of peak, {describe(w)}"


def cpu_baseline(w, q, k, v, desc, budget_s):
    """Time the fp64 oracle (as it stands) on whole heads of the workload until
    ``budget_s`` seconds of CPU work have accumulated; scale to TFLOP/s with
    the metric's FLOP count of the heads done."""
    import numpy as np
    import oracle
    from tests.helpers import to_f64
    from scaled_dot_product_09_amd.workload import metric_flops
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    G = w.Hq // w.Hkv
    done, elapsed = 0, 0.0
    for b in range(w.B):
        for hq in range(w.Hq):
            g = hq // G
            qh = to_f64(q[b:b + 1, :, hq:hq + 1], w.dtype, desc[0])
            kh = to_f64(k[b:b + 1, :, g:g + 1], w.dtype, desc[1])
            vh = to_f64(v[b:b + 1, :, g:g + 1], w.dtype, desc[2])
            t0 = time.perf_counter()
            oracle.sdpa(qh, kh, vh, scale=w.scale, causal=w.causal)
            elapsed += time.perf_counter() - t0
            done += 1
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    flops = metric_flops(1, done, w.Sq, w.Skv, w.D, w.causal)
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
    except OSError:
        pass
    full = " (the oracle forms the whole matrix: twice the counted causal FLOPs)" if w.causal else ""
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hq} (batch, query head) pairs of the same workload, full "
                      f"Sq x Skv each{full}, fp64 numpy on {threads} BLAS threads, {elapsed:.1f} s; "
                      f"host: {os.cpu_count()} CPUs, {model}"}


def cpu_baseline_bwd(w, q, k, v, desc, budget_s):
    """Time the fp64 backward oracle (as it stands) on whole (batch, KV-head
    group) units of a backward workload (the group's query heads with their
    KV head, the workload's own dout) until ``budget_s`` seconds of CPU work
    have accumulated; scale to TFLOP/s with the metric's backward FLOP count
    of the heads done."""
    import oracle
    from tests.helpers import to_f64
    from scaled_dot_product_09_amd.workload import bwd_metric_flops, make_dout
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    g = make_dout(w)
    gdt, gdesc = ("e5m2", g[1]) if w.dtype == "e4m3" else (w.dtype, 1.0)
    g = g[0] if w.dtype == "e4m3" else g
    G = w.Hq // w.Hkv
    done, elapsed = 0, 0.0
    for b in range(w.B):
        for hk in range(w.Hkv):
            hs = slice(hk * G, (hk + 1) * G)
            qh = to_f64(q[b:b + 1, :, hs], w.dtype, desc[0])
            kh = to_f64(k[b:b + 1, :, hk:hk + 1], w.dtype, desc[1])
            vh = to_f64(v[b:b + 1, :, hk:hk + 1], w.dtype, desc[2])
            gh = to_f64(g[b:b + 1, :, hs], gdt, gdesc)
            t0 = time.perf_counter()
            oracle.sdpa_backward(qh, kh, vh, gh, scale=w.scale, causal=w.causal)
            elapsed += time.perf_counter() - t0
            done += G
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    flops = bwd_metric_flops(1, done, w.Sq, w.Skv, w.D, w.causal)
    full = " (the oracle forms the whole matrices: twice the counted causal FLOPs)" if w.causal else ""
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hq} (batch, query head) pairs of the same workload, whole KV-head "
                      f"groups, full Sq x Skv each{full}, fp64 numpy backward on {threads} BLAS threads, "
                      f"{elapsed:.1f} s; host: {os.cpu_count()} CPUs"}


def time_workload(w, steps, warmup, rotate=True, settle_s=SETTLE_S):
    import torch
    from scaled_dot_product_09_amd import attn, workload
    dev = torch.device("cuda:0")
    q, k, v, desc = workload.make_inputs(w)
    nsets = N_BUFFER_SETS if rotate else 1
    sets = []
    for i in range(nsets):
        qd, kd, vd = (workload.to_layout(x.to(dev), w.layout) for x in (q, k, v))
        od = workload.to_layout(torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "e4m3" else q.dtype,
                                            device=dev), w.layout)
        sets.append((qd, kd, vd, od))
    fp8 = w.dtype == "e4m3"
    stream = torch.cuda.current_stream(dev)

    ws = None
    if w.n_split is not None:
        n_split = w.n_split
        if n_split == "auto":
            n_split = attn.attn_split_suggest(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, attn.CAUSAL_CODE[w.causal])
        ws = torch.empty(max(attn.attn_split_workspace(w.B, w.Hq, w.Sq, w.D, n_split), 16), dtype=torch.uint8,
                         device=dev)

    def step(i):
        qd, kd, vd, od = sets[i % nsets]
        attn.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=od,
                 descales=desc if fp8 else None, stream=stream.cuda_stream,
                 n_split=n_split if ws is not None else None, workspace=ws)

    if w.scaling == "delayed":
        # One delayed-scaling FP8 step: cast bf16 q, k, v to E4M3 with each
        # tensor's device-side state, the forward reading the three factors
        # on the device, one update of the three states. No host read-back.
        bf = [torch.from_numpy(x).to(torch.bfloat16).to(dev)
              for x in workload.draw_normal(w.seed, [(w.B, w.Sq, w.Hq, w.D), (w.B, w.Skv, w.Hkv, w.D),
                                                     (w.B, w.Skv, w.Hkv, w.D)])]
        states = attn.fp8_states(3, attn.ATTN_FP8_E4M3)
        codes = [torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev) for x in bf]
        od = torch.empty(bf[0].shape, dtype=torch.bfloat16, device=dev)

        def step(i):  # noqa: F811
            for x, c, j in zip(bf, codes, range(3)):
                attn.fp8_quantize(x, states[j], attn.ATTN_FP8_E4M3, out=c, stream=stream.cuda_stream)
            attn.fwd_fp8_dev(*codes, [states[0], states[1], states[2]], causal=w.causal, scale=w.scale, out=od,
                             stream=stream.cuda_stream)
            attn.fp8_update(states, stream=stream.cuda_stream)

    if w.direction == "bwd":
        # Backward: the forward's out and lse are made once per input set,
        # outside the timed region; a step is one attn_bwd (attn_bwd_fp8 for
        # E4M3 inputs with an E5M2 gradient) call.
        g = workload.make_dout(w)
        bdesc = None
        if fp8:
            g, gdesc = g
            bdesc = (*desc, gdesc)
        g = g.to(dev)
        bsets = []
        for qd, kd, vd, od in sets:
            od, lse = attn.fwd_lse(qd, kd, vd, causal=w.causal, scale=w.scale, out=od,
                                   descales=desc if fp8 else None)
            bsets.append((qd, kd, vd, od, lse, torch.empty_like(od), torch.empty(kd.shape, dtype=od.dtype, device=dev),
                          torch.empty(vd.shape, dtype=od.dtype, device=dev)))
        need = (attn.attn_bwd_fp8_workspace(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D) if fp8
                else attn.attn_bwd_workspace(w.B, w.Hq, w.Sq))
        bws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def step(i):  # noqa: F811
            qd, kd, vd, od, lse, dq, dk, dv = bsets[i % nsets]
            attn.bwd(qd, kd, vd, od, g, lse, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=bws,
                     stream=stream.cuda_stream, descales=bdesc)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # After idle the GPU needs some tens of milliseconds of load to reach its
    # sustained clock (the first ~30 headline launches run up to 25 % slower):
    # keep stepping, untimed, until at least settle_s of work has run.
    settle = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for i in range(8):
            step(warmup + settle + i)
        settle += 8
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    total = ev[0].elapsed_time(ev[steps])
    return {"ms_per_step": total / steps, "median_ms": per[len(per) // 2], "min_ms": per[0],
            "settle_steps": settle, "inputs": (q, k, v, desc), "n_split": n_split if ws is not None else 1}


def result_line(w, t, steps, warmup, n_gpus, cpu=None, warm=None):
    from scaled_dot_product_09_amd.workload import workload_flops, io_bytes
    flops = workload_flops(w)
    ms = t["ms_per_step"]
    tflops = flops / (ms * 1e-3) / 1e12
    # The products' arithmetic type: the FP8 backward widens its codes and
    # multiplies in bf16.
    compute = "bf16" if (w.direction == "bwd" and w.dtype == "e4m3") else w.dtype
    peak = PEAK_TFLOPS[compute]
    nbytes = io_bytes(w)
    gbps = nbytes / (ms * 1e-3) / 1e9
    # Below the ridge point (peak flop/s over peak HBM bytes/s) the attention
    # kernel is bound by HBM, not by the matrix cores. The attention's own
    # bytes decide (a delayed-scaling step's casts are separate HBM-bound
    # kernels beside the dominant attention kernel).
    from dataclasses import replace
    attn_bytes = io_bytes(replace(w, scaling="amax"))
    hbm_bound = flops / attn_bytes < peak * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    else:
        roof = {"bound": PEAK_KIND[compute], "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4)}
    roof.update({"traffic": load_traffic(w), "algorithmic_bytes": nbytes})
    line = {
        "metric": metric_name(w), "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": n_gpus,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Skv": w.Skv,
                   "D": w.D, "causal": w.causal, "input_dtype": w.dtype, "output_dtype": w.out_dtype,
                   "parallelism": "single GPU", "rotating_input_sets": N_BUFFER_SETS, "layout": w.layout,
                   "direction": w.direction},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "median_ms": round(t["median_ms"], 5), "min_ms": round(t["min_ms"], 5),
        "settle_steps": t["settle_steps"],
        "hbm_gbps": round(gbps, 1),
        "roofline": roof,
    }
    if t.get("n_split", 1) != 1:
        line["config"]["n_split"] = t["n_split"]
        line["config"]["entry_point"] = "attn_fwd_split"
    if warm is not None:
        line["warm_single_set_ms"] = round(warm["ms_per_step"], 5)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="named workload (default: the GQA headline)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--sweep-out", default=None, help="also time every named workload, JSONL to this file")
    ap.add_argument("--sweep-cpu-budget", type=float, default=3.0,
                    help="seconds of oracle time for each sweep line's cpu_baseline (0: none)")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed steps after the warmup steps (clock settle)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB (untimed), a "
                         "reference dispatch of known size for scaling hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs each attention call on a single MI355X "
              "and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from scaled_dot_product_09_amd import workload
    name = args.workload or workload.HEADLINE
    w = workload.WORKLOADS[name]

    if args.copy_ref_mib:
        import torch
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t = time_workload(w, args.steps, args.warmup, rotate=True, settle_s=args.settle_s)
    warm = time_workload(w, args.steps, args.warmup, rotate=False, settle_s=args.settle_s)
    cpu = None
    if not args.no_cpu and w.scaling == "amax":
        q, k, v, desc = t["inputs"]
        cpu = (cpu_baseline if w.direction == "fwd" else cpu_baseline_bwd)(w, q, k, v, desc, args.cpu_budget)
    line = result_line(w, t, args.steps, args.warmup, 1, cpu=cpu, warm=warm)

    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            for n, wi in workload.WORKLOADS.items():
                ti = time_workload(wi, args.steps, args.warmup, rotate=True, settle_s=args.settle_s)
                ci = None
                if args.sweep_cpu_budget > 0 and wi.scaling == "amax":
                    qi, ki, vi, di = ti["inputs"]
                    if wi.direction == "fwd":
                        ci = cpu_baseline(wi, qi, ki, vi, di, args.sweep_cpu_budget)
                    else:
                        ci = cpu_baseline_bwd(wi, qi, ki, vi, di, args.sweep_cpu_budget)
                f.write(json.dumps(result_line(wi, ti, args.steps, args.warmup, 1, cpu=ci)) + "\n")
                f.flush()
                print(f"sweep {n}: {ti['ms_per_step']:.4f} ms", file=sys.stderr, flush=True)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
