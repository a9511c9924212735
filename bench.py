"""Benchmark of the W4A16 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode|mid|prefill|actorder|tiny]

A step is one forward pass of the hot path over every (shape, M) case of the
chosen workload: for each case one w4a16_linear call (host validation, kernel
selection, fused dequantize + GEMM, epilogue) on activations and weights that
are already resident in HBM.  The timed launches are recorded into a HIP
graph and replayed (as a serving loop would), so the ~5 us host cost of a
Python call does not starve the GPU between short decode kernels; --eager
times direct launches instead.  The one-time repacks (AWQ -> standard ->
tile layout) are timed separately and reported under "repack".

Weight buffers are rotated over enough copies that every launch reads its
weights from HBM (the working set exceeds the 256 MB Infinity Cache).

Prints ONE JSON line.  ``value`` is packed-weight GB/s of the whole step
(sum of K*N/2 over the cases / step time); ``roofline`` is for the GEMM
kernel with achieved = algorithmic bytes per launch / HIP-event launch time;
``cpu_baseline`` times the CPU oracle on a bounded sample of the workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM TFLOPS + packed-weight HBM GB/s (% roofline), M=1..8192"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
ROTATE_BYTES = 512 << 20       # working set per shape, > 256 MB MALL
COPY_PROBE_BYTES = 256 << 20   # plain device copy used to calibrate byte counters


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="decode", choices=["tiny", "decode", "mid", "prefill", "actorder", "moe"])
    p.add_argument("--reps", type=int, default=0, help="launches per case for the per-kernel timing (0 = auto)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--group-size", type=int, default=0, choices=[0, 32, 64, 128, -1],
                   help="run the workload's shapes with this group size instead (0 = the workload's own)")
    p.add_argument("--compare", action="store_true",
                   help="also time the unfused path (dense dequantization kernel, then torch.matmul) per case")
    p.add_argument("--eager", action="store_true",
                   help="time direct launches instead of HIP-graph replays (host launch cost included)")
    return p.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_decode_hbm_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "weight_only_int4_gptq_amd", "csrc", "w4_gemm.hip")


def measured_traffic():
    """HBM bytes per decode GEMM launch from the committed rocprofv3 counter
    summary, or None when the GEMM source changed since it was measured."""
    import hashlib
    try:
        fields = dict(line.split(": ", 1) for line in open(TRAFFIC_PROFILE).read().splitlines()
                      if line and not line.startswith("#") and ": " in line)
        cur = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != cur:
        return None
    return int(float(fields["per_launch_traffic_bytes"]))


def _to_dev(torch, a):
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case_bytes(c, M):
    """Algorithmic HBM bytes of one launch: packed weights + scales + zeros +
    x + y (+ perm)."""
    w = c.K * c.N // 2
    s = c.G * c.N * 2
    z = c.G * c.N // 2 if c.has_zeros else 0
    x = M * c.K * 2
    y = M * c.N * 2
    p = c.K * 4 if c.has_gidx else 0
    return w, w + s + z + x + y + p


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_int4_gptq_amd as W
    from synthetic import CONFIGS, make_acts, make_layer_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    W.lib()
    if args.config == "moe":
        return main_moe(args, torch, W)
    cfg_id = {"tiny": 1, "decode": 2, "mid": 3, "prefill": 4, "actorder": 5}[args.config]
    cases = [c for c in CONFIGS if c.cfg_id == cfg_id]
    if args.group_size:
        import dataclasses
        cases = [dataclasses.replace(c, group_size=args.group_size, has_gidx=c.has_gidx and args.group_size != -1)
                 for c in cases]
    stream = torch.cuda.current_stream()

    # ---- one-time repack (timed separately) and rotated weight copies ----
    layers = []
    repack = []
    for c in cases:
        Lw = make_layer_inputs(c)
        dev = {k: _to_dev(torch, v) for k, v in Lw.items()}
        lyr = W.W4A16Linear(c.K, c.N, c.group_size, c.has_zeros, c.has_gidx, c.dtype, c.fmt)
        lyr.process_weights_after_loading(dev["qweight"], dev["qzeros"], dev["scales"], dev["g_idx"])  # warm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lyr.process_weights_after_loading(dev["qweight"], dev["qzeros"], dev["scales"], dev["g_idx"])
        e1.record(stream)
        torch.cuda.synchronize()
        rp_ms = e0.elapsed_time(e1)
        repack.append({"shape": [c.K, c.N], "ms": round(rp_ms, 4),
                       "packed_GBps": round((c.K * c.N / 2) / (rp_ms * 1e-3) / 1e9, 1)})
        t = lyr.tiled
        per_set = sum(v.numel() * v.element_size() for v in t.values() if v is not None)
        R = max(2, math.ceil(ROTATE_BYTES / per_set))
        sets = [t] + [{k: (v.clone() if v is not None else None) for k, v in t.items()} for _ in range(R - 1)]
        del dev
        layers.append((c, lyr, sets))
    torch.cuda.synchronize()

    # ---- activations / outputs per case ----
    runs = []
    for c, lyr, sets in layers:
        for M in c.Ms:
            x = make_acts(c, M)
            xd = _to_dev(torch, x)
            yd = torch.empty((M, c.N), dtype=xd.dtype, device="cuda")
            ws_b = W.w4_workspace_size(lyr.layer, M)
            ws = torch.zeros((max(ws_b, 1),), dtype=torch.uint8, device="cuda")
            runs.append(dict(c=c, M=M, lyr=lyr, sets=sets, x=xd, y=yd, ws=ws, ws_b=ws_b, i=0,
                             kernel=lyr.kernel_name(M)))

    def launch(r):
        # the current stream: the capture stream while a HIP graph is recorded
        t = r["sets"][r["i"] % len(r["sets"])]
        r["i"] += 1
        W.w4a16_linear(r["lyr"].layer, r["M"], r["x"], t["qweight"], t["scales"], t["qzeros"], t["perm"], None,
                       r["y"], r["ws"] if r["ws_b"] else None, r["ws_b"], torch.cuda.current_stream())

    def step():
        for r in runs:
            launch(r)

    def timed(fn, count):
        """Milliseconds for the launches that fn() enqueues, HIP events on the
        launch stream.  By default fn's launches are recorded once into a HIP
        graph, which is replayed once untimed (upload) and once timed, so the
        host's per-call cost (Python, ctypes, validation: ~5 us) does not
        starve the GPU between short kernels, as in a serving loop."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.eager:
            torch.cuda.synchronize()
            e0.record(stream)
            fn(count)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(count)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1)

    # ---- per-kernel timing: HIP events on the launch stream ----
    per_case = []
    for r in runs:
        c, M = r["c"], r["M"]
        reps = args.reps or max(len(r["sets"]), 40)
        for _ in range(5):
            launch(r)
        torch.cuda.synchronize()
        us = timed(lambda n: [launch(r) for _ in range(n)], reps) * 1e3 / reps
        wb, tb = case_bytes(c, M)
        flops = 2.0 * M * c.K * c.N
        per_case.append(dict(K=c.K, N=c.N, M=M, kernel=r["kernel"], us=round(us, 3),
                             weight_GBps=round(wb / (us * 1e-6) / 1e9, 1),
                             total_GBps=round(tb / (us * 1e-6) / 1e9, 1),
                             TFLOPS=round(flops / (us * 1e-6) / 1e12, 2),
                             pct_hbm=round(100 * tb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                             pct_mfma=round(100 * flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 1),
                             _wb=wb, _tb=tb, _flops=flops, _us=us))

    # ---- copy of known size (not timed): the reference for the HBM byte
    # counters when this run is profiled (FETCH_SIZE / WRITE_SIZE) ----
    src = torch.empty((COPY_PROBE_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # ---- the timed steps ----
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = timed(lambda n: [step() for _ in range(n)], args.steps) / args.steps
    wall = time.perf_counter() - t0

    wbytes_step = sum(case_bytes(r["c"], r["M"])[0] for r in runs)
    flops_step = sum(2.0 * r["M"] * r["c"].K * r["c"].N for r in runs)
    value = wbytes_step / (ms_step * 1e-3) / 1e9

    # roofline of the GEMM kernel: algorithmic bytes (or flops) / launch time
    sum_tb = sum(p["_tb"] for p in per_case)
    sum_fl = sum(p["_flops"] for p in per_case)
    sum_us = sum(p["_us"] for p in per_case)
    hbm_bound = (sum_fl / (sum_tb)) < (MFMA_F16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        ach = sum_tb / (sum_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        ach = sum_fl / (sum_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    if hbm_bound and args.config == "decode":
        roof["traffic"] = measured_traffic()
    roof["kernel"] = sorted({p["kernel"] for p in per_case})
    roof["per_launch_bytes_avg"] = round(sum_tb / len(per_case))
    roof["avg_launch_us"] = round(sum_us / len(per_case), 3)

    unfused = compare_unfused(torch, runs, per_case, stream) if args.compare else None

    cpu = None if args.no_cpu else cpu_baseline(cases, args.cpu_seconds)

    for p in per_case:
        for k in ("_wb", "_tb", "_flops", "_us"):
            p.pop(k)
    c0 = cases[0]
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if c0.dtype == "fp16" else "bf16",
        "data": "synthetic (seeded uniform int4 codes/zeros, uniform scales, N(0,1) activations)",
        "config": {
            "workload": f"{args.config}: " + ", ".join(f"(K={c.K},N={c.N})" for c in cases)
                        + f" x M in {list(c0.Ms)}; {c0.fmt.upper()} g={c0.group_size}"
                        + (" zeros" if c0.has_zeros else " symmetric") + (" act-order" if c0.has_gidx else ""),
            "cases": len(runs), "act_dtype": c0.dtype, "weight_rotation_MiB": ROTATE_BYTES >> 20,
            "copy_probe_MiB": COPY_PROBE_BYTES >> 20,
        },
        "timing": ("eager launches" if args.eager else
                   "HIP graph of the timed launches (one untimed replay uploads it, one replay is timed)"),
        "tflops_step": round(flops_step / (ms_step * 1e-3) / 1e12, 3),
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "dequant_then_gemm": unfused,
        "cpu_baseline": cpu,
        "per_case": per_case,
        "repack": repack,
    }
    print(json.dumps(out), flush=True)


# Mixture-of-experts workload (not one of the five layer workloads): the fused
# gate/up projection of a Mixtral-8x7B-class MoE layer, 8 experts of
# (K, N) = (4096, 28672), fp16 AWQ g = 128 with zero points, tokens routed
# top-2 by a seeded random router; rows per step 32 (16 decode tokens),
# 512 (256 tokens) and 4096 (2048 prefill tokens).
MOE_E, MOE_K, MOE_N, MOE_TOKENS, MOE_TOPK = 8, 4096, 28672, (16, 256, 2048), 2


def main_moe(args, torch, W):
    from synthetic import normal_acts, random_words, seeded, uniform_scales
    stream = torch.cuda.current_stream()
    E, K, N = MOE_E, MOE_K, MOE_N
    G = K // 128
    experts = []
    for e in range(E):
        rng = seeded(6, K, N, e)
        experts.append((random_words(rng, (K, N // 8)), random_words(rng, (G, N // 8)),
                        uniform_scales(rng, (G, N), 0.002, 0.02, "fp16")))
    moe = W.W4A16MoELinear(E, K, N, 128, True, "fp16", "awq")
    moe.process_weights_after_loading([tuple(_to_dev(torch, a) for a in ex) for ex in experts])
    t0 = moe.tiled
    per_set = sum(v.numel() * v.element_size() for v in t0.values() if v is not None)
    R = max(2, math.ceil(ROTATE_BYTES / per_set))
    sets = [t0] + [{k: (v.clone() if v is not None else None) for k, v in t0.items()} for _ in range(R - 1)]
    runs = []
    for T in MOE_TOKENS:
        rng = seeded(7, T)
        choice = np.stack([rng.choice(E, size=MOE_TOPK, replace=False) for _ in range(T)])  # top-2 experts
        counts = np.bincount(choice.reshape(-1), minlength=E)
        offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        rows = int(offs[-1])
        x = _to_dev(torch, normal_acts(seeded(8, rows, K), (rows, K), "fp16"))
        y = torch.empty((rows, N), dtype=torch.float16, device="cuda")
        runs.append(dict(T=T, rows=rows, max_rows=int(counts.max()), offs=_to_dev(torch, offs), x=x, y=y,
                         counts=counts.tolist(), i=0))

    def launch(r):
        t = sets[r["i"] % len(sets)]
        r["i"] += 1
        W.w4a16_moe_linear(moe.layer, E, r["rows"], r["max_rows"], r["x"], r["offs"], t["qweight"], t["scales"],
                           t["qzeros"], None, r["y"], torch.cuda.current_stream())

    def timed(fn, count):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(count)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    wbytes = E * K * N // 2
    per_case = []
    for r in runs:
        for _ in range(3):
            launch(r)
        torch.cuda.synchronize()
        reps = 20 if r["rows"] >= 1024 else 60
        us = timed(lambda n: [launch(r) for _ in range(n)], reps) * 1e3 / reps
        tb = wbytes + E * G * N * 2 + E * G * N // 2 + r["rows"] * (K + N) * 2
        fl = 2.0 * r["rows"] * K * N
        per_case.append(dict(tokens=r["T"], rows=r["rows"], rows_per_expert=r["counts"], us=round(us, 3),
                             weight_GBps=round(wbytes / (us * 1e-6) / 1e9, 1), TFLOPS=round(fl / (us * 1e-6) / 1e12, 2),
                             _tb=tb, _fl=fl, _us=us))

    def step():
        for r in runs:
            launch(r)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0w = time.perf_counter()
    ms_step = timed(lambda n: [step() for _ in range(n)], args.steps) / args.steps
    wall = time.perf_counter() - t0w
    value = len(runs) * wbytes / (ms_step * 1e-3) / 1e9
    sum_tb = sum(p["_tb"] for p in per_case)
    sum_fl = sum(p["_fl"] for p in per_case)
    sum_us = sum(p["_us"] for p in per_case)
    if sum_fl / sum_tb < (MFMA_F16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9):
        ach = sum_tb / (sum_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        ach = sum_fl / (sum_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    roof["kernel"] = ["w4a16_moe_linear (wide kernel, grouped)"]
    roof["avg_launch_us"] = round(sum_us / len(per_case), 3)
    cpu = None
    if not args.no_cpu:
        import oracle as O
        qw, qz, sc = experts[0]
        xs = normal_acts(seeded(9, 4, K), (4, K), "fp16")
        tc = time.perf_counter()
        O.reference_moe(xs, np.array([0, 4]), "awq", "fp16", [experts[0]], 128)
        dt = time.perf_counter() - tc
        cpu = {"value": round((K * N // 2) / dt / 1e9, 4), "unit": "GB/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": "one expert (K=4096, N=28672) on 4 rows", "seconds": round(dt, 2)}
    for p in per_case:
        for k in ("_tb", "_fl", "_us"):
            p.pop(k)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded uniform int4 codes/zeros, uniform scales, N(0,1) activations, random top-2 routing)",
        "config": {"workload": f"moe: E={E} experts of (K={K},N={N}) AWQ g=128 zeros, top-{MOE_TOPK} routing of "
                               f"{list(MOE_TOKENS)} tokens", "cases": len(runs), "act_dtype": "fp16",
                   "weight_rotation_MiB": ROTATE_BYTES >> 20},
        "timing": "HIP graph of the timed launches (one untimed replay uploads it, one replay is timed)",
        "wall_s_timed": round(wall, 3), "roofline": roof, "cpu_baseline": cpu, "per_case": per_case,
    }
    print(json.dumps(out), flush=True)


def compare_unfused(torch, runs, per_case, stream):
    """The unfused path the pages describe for large batches: the library's
    dense dequantization kernel writes W [K, N] in the activation dtype, then
    torch.matmul (the vendor GEMM) computes x W.  Each part is timed with HIP
    events over back-to-back direct launches, per case, next to the fused
    kernel's time from the roofline timing."""
    out = []
    for r, pc in zip(runs, per_case):
        lyr, M = r["lyr"], r["M"]
        w = torch.empty((lyr.K, lyr.N), dtype=r["x"].dtype, device="cuda")
        t = r["sets"][0]

        def dq():
            import weight_only_int4_gptq_amd as W
            W.w4_dequant_dense(lyr.layer, t["qweight"], t["scales"], t["qzeros"], t["perm"], w, stream)

        def mm():
            torch.matmul(r["x"], w, out=r["y"])

        res = {}
        for name, fn in (("dequant_us", dq), ("gemm_us", mm)):
            reps = 20 if M >= 1024 else 50
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / reps
        tot = res["dequant_us"] + res["gemm_us"]
        out.append({"K": lyr.K, "N": lyr.N, "M": M, "dequant_us": round(res["dequant_us"], 3),
                    "gemm_us": round(res["gemm_us"], 3), "unfused_us": round(tot, 3), "fused_us": pc["us"],
                    "fused_speedup": round(tot / pc["us"], 3)})
        del w
    return out


def cpu_baseline(cases, seconds):
    """The CPU oracle, as it stands, on a bounded sample of the workload:
    whole-layer reference (unpack, order fix, float64 dequant, float64 matmul)
    for the workload's cases in order until ``seconds`` of CPU time are spent.
    Value in the metric's unit (packed-weight GB/s)."""
    import oracle as O
    from synthetic import make_acts, make_layer_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    done, wbytes, spent = [], 0, 0.0
    for _ in range(8):  # passes over the workload until `seconds` of CPU time are spent
        for c in cases:
            Lw = make_layer_inputs(c)
            for M in c.Ms:
                x = make_acts(c, M)
                t0 = time.perf_counter()
                O.reference_linear(x, c.fmt, c.dtype, Lw["qweight"], Lw["qzeros"], Lw["scales"], c.group_size,
                                   g_idx=Lw["g_idx"])
                dt = time.perf_counter() - t0
                spent += dt
                wbytes += c.K * c.N // 2
                done.append(f"(K={c.K},N={c.N},M={M})")
                if spent >= seconds:
                    break
            if spent >= seconds:
                break
        if spent >= seconds:
            break
    return {"value": round(wbytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} whole-layer oracle calls cycling through the cases "
                      + " ".join(dict.fromkeys(done)), "seconds": round(spent, 2)}


if __name__ == "__main__":
    main()
