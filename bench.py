"""Benchmark of the W4A16 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--config all|decode|tiny|mid|prefill|actorder|prefill_bf16|w4a8|moe] [--compare]
                    [--group-size G]

A step is one forward pass of the hot path over every (shape, M) case of the
decode workload (7B-class layers, M = 1, 4, 16): for each case one
w4a16_linear call (host validation, kernel selection, fused dequantize +
GEMM, epilogue) on activations and weights already resident in HBM.  K steps
are recorded into a HIP graph; one untimed replay uploads it and one replay
is timed (a serving loop replays graphs the same way, so the ~5 us host cost
of a Python call does not starve the GPU between short decode kernels;
--eager times direct launches instead).  ``value`` is packed-weight GB/s of
that step.

With ``--config all`` (the default) the line also carries one block per
workload (decode, tiny, mid-batch, prefill, act-order, and the prefill shapes
as bf16 GPTQ layers), so the metric is
covered over M = 1..8192: each case is timed alone as the median of five
replays of a graph of back-to-back launches, and each block reports its
roofline (HBM-bound cases against 8 TB/s on algorithmic bytes, MFMA-bound
cases against the dense fp16/bf16 peak on 2 M K N flops).  A last block,
"w4a8", runs the decode and prefill layers with FP8-E4M3 activations
(w4a8_linear: activation quantization plus the int4 x fp8 GEMM, per call),
its MFMA-bound cases priced against the dense fp8 peak.

Weight buffers are rotated over enough copies that every launch reads its
weights from HBM (the working set exceeds the 256 MB Infinity Cache).  The
one-time repacks (AWQ -> standard -> tile layout) are timed separately.
``cpu_baseline`` times the CPU oracle's three phases (unpack + order fix +
standard repack, float64 dequantization, float64 matmul) on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM TFLOPS + packed-weight HBM GB/s (% roofline), M=1..8192"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
MFMA_F8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
ROTATE_BYTES = 512 << 20       # working set per shape, > 256 MB MALL
COPY_PROBE_BYTES = 256 << 20   # plain device copy used to calibrate byte counters
REPLAYS = 5                    # per-case timing: median of this many graph replays
WORKLOADS = ("decode", "tiny", "mid", "prefill", "actorder", "prefill_bf16", "w4a8")
FLOOR_WORKLOADS = ("decode", "tiny")  # the HBM-bound ones that --floor covers
FLOOR_SWEEP_WGS = (256, 512, 1024, 2048, 4096)
FLOOR_TAGS = 15      # empty_kernel<0..14> / stream_read<0..14> name the floor cases
MARKER_TAG = 15      # empty_kernel<15> on one wave: the --markers case separator
FLOOR_SWEEP_THREADS = (256, 512, 1024)
CFG_ID = {"tiny": 1, "decode": 2, "mid": 3, "prefill": 4, "actorder": 5, "prefill_bf16": 6}
# W4A8-fp8 workload: the decode and prefill layers with FP8-E4M3 activations
# (static per-tensor scale), quantization included in every call
W4A8_CFGS = (2, 4)
W4A8_X_SCALE = 0.01171875


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default="all", choices=["all", *WORKLOADS, "moe"])
    p.add_argument("--reps", type=int, default=0, help="launches per case graph (0 = auto)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--group-size", type=int, default=0, choices=[0, 32, 64, 128, -1],
                   help="run the workloads' shapes with this group size instead (0 = their own)")
    p.add_argument("--compare", action="store_true",
                   help="also time the unfused path (dense dequantization kernel, then torch.matmul) per case")
    p.add_argument("--floor", action="store_true",
                   help="per HBM-bound case, also time a plain streaming read of the case's algorithmic bytes "
                        "and an empty kernel, both on the GEMM's own grid (libw4floor)")
    p.add_argument("--markers", action="store_true",
                   help="launch a one-wave empty kernel (empty_kernel<15>, libw4floor) before each case and after "
                        "the last, outside every timed region, so that a profiler trace splits into cases")
    p.add_argument("--eager", action="store_true",
                   help="time direct launches instead of HIP-graph replays (host launch cost included)")
    return p.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_decode_hbm_traffic.txt")
CSRC = os.path.join(ROOT, "weight_only_int4_gptq_amd", "csrc")


def source_digest():
    """sha256 over the library's sources (csrc/*.h, *.hip, *.cpp: name and
    contents, sorted by name): the version that a stored profile was taken of."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(CSRC, "*.hip"))
                    + glob.glob(os.path.join(CSRC, "*.cpp"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode GEMM launch from the committed rocprofv3 counter
    summary, or None when the library's sources changed since it was measured."""
    try:
        fields = dict(line.split(": ", 1) for line in open(TRAFFIC_PROFILE).read().splitlines()
                      if line and not line.startswith("#") and ": " in line)
        cur = source_digest()
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
    """(packed-weight bytes, algorithmic HBM bytes) of one launch: packed
    weights + scales + zeros + x + y (+ perm)."""
    w = c.K * c.N // 2
    s = c.G * c.N * 2
    z = c.G * c.N // 2 if c.has_zeros else 0
    x = M * c.K * 2
    y = M * c.N * 2
    p = c.K * 4 if c.has_gidx else 0
    return w, w + s + z + x + y + p


def roofline_of(cases, mfma_peak=MFMA_F16_PEAK_TFLOPS):
    """Roofline objects of a set of timed cases, one per bound: a case whose
    flop per algorithmic byte is below the ridge (MFMA peak / HBM peak) is
    HBM-bound, else MFMA-bound.  achieved = algorithmic bytes (flops) of the
    cases / the sum of their per-launch times."""
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    out = []
    for bound in ("hbm", "mfma"):
        sel = [p for p in cases if (p["_flops"] / p["_tb"] < ridge) == (bound == "hbm")]
        if not sel:
            continue
        us = sum(p["_us"] for p in sel)
        if bound == "hbm":
            ach = sum(p["_tb"] for p in sel) / (us * 1e-6) / 1e9
            r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
        else:
            ach = sum(p["_flops"] for p in sel) / (us * 1e-6) / 1e12
            r = {"bound": "mfma", "achieved": round(ach, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                 "frac": round(ach / mfma_peak, 4), "traffic": None}
        r["kernel"] = sorted({p["kernel"] for p in sel})
        r["cases"] = [f"K={p['K']} N={p['N']} M={p['M']}" for p in sel]
        r["per_launch_bytes_avg"] = round(sum(p["_tb"] for p in sel) / len(sel))
        r["per_launch_flops_avg"] = round(sum(p["_flops"] for p in sel) / len(sel))
        r["avg_launch_us"] = round(us / len(sel), 3)
        out.append(r)
    return out


class Bench:
    def __init__(self, args, torch, W):
        self.args, self.torch, self.W = args, torch, W
        self.stream = torch.cuda.current_stream()

    # ---- timing -------------------------------------------------------------
    def timed(self, fn, count, replays=1):
        """Milliseconds for the launches that fn(count) enqueues, HIP events on
        the launch stream.  By default fn's launches are recorded once into a
        HIP graph, which is replayed once untimed (upload) and then ``replays``
        times, each timed on its own; the median is returned."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if self.args.eager:
            ts = []
            for _ in range(replays):
                torch.cuda.synchronize()
                e0.record(self.stream)
                fn(count)
                e1.record(self.stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return statistics.median(ts)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(count)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(replays):
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        del g
        return statistics.median(ts)

    def marker(self):
        """With --markers: one empty one-wave kernel (empty_kernel<15>) on
        the current stream, a case boundary in a profiler trace."""
        if not self.args.markers:
            return
        import ctypes
        if not hasattr(self, "_floor_lib"):
            F = ctypes.CDLL(os.path.join(ROOT, "weight_only_int4_gptq_amd", "libw4floor.so"))
            F.w4floor_empty.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_uint32, ctypes.c_int,
                                        ctypes.c_void_p]
            self._floor_lib = F
        g = (ctypes.c_uint32 * 3)(1, 1, 1)
        e = self._floor_lib.w4floor_empty(g, 64, MARKER_TAG, self.torch.cuda.current_stream().cuda_stream)
        assert e == 0, f"w4floor_empty: hip error {e}"

    # ---- workloads ----------------------------------------------------------
    def setup(self, name):
        """Layers (repacked, weight copies for rotation) and per-case buffers."""
        import dataclasses
        torch, W = self.torch, self.W
        from synthetic import CONFIGS, make_acts, make_layer_inputs
        fp8 = name == "w4a8"
        cases = [c for c in CONFIGS if (c.cfg_id in W4A8_CFGS if fp8 else c.cfg_id == CFG_ID[name])]
        gs = self.args.group_size
        if gs:
            cases = [dataclasses.replace(c, group_size=gs, has_gidx=c.has_gidx and gs != -1) for c in cases]
        layers, repack = [], []
        for c in cases:
            Lw = make_layer_inputs(c)
            dev = {k: _to_dev(torch, v) for k, v in Lw.items()}
            lyr = W.W4A16Linear(c.K, c.N, c.group_size, c.has_zeros, c.has_gidx, c.dtype, c.fmt)
            lyr.process_weights_after_loading(dev["qweight"], dev["qzeros"], dev["scales"], dev["g_idx"])  # warm
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            lyr.process_weights_after_loading(dev["qweight"], dev["qzeros"], dev["scales"], dev["g_idx"])
            e1.record(self.stream)
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
        runs = []
        for c, lyr, sets in layers:
            for M in c.Ms:
                xd = _to_dev(torch, make_acts(c, M))
                yd = torch.empty((M, c.N), dtype=xd.dtype, device="cuda")
                ws_b = W.w4a8_workspace_size(lyr.layer, M) if fp8 else W.w4_workspace_size(lyr.layer, M)
                ws = torch.zeros((max(ws_b, 1),), dtype=torch.uint8, device="cuda")
                runs.append(dict(c=c, M=M, lyr=lyr, sets=sets, x=xd, y=yd, ws=ws, ws_b=ws_b, i=0, fp8=fp8,
                                 xs=torch.tensor([W4A8_X_SCALE], dtype=torch.float32, device="cuda"),
                                 kernel=("w4a8_quantize + " + W.w4a8_kernel_name(lyr.layer, M)) if fp8
                                 else lyr.kernel_name(M)))
        return cases, runs, repack

    def launch(self, r):
        # the current stream: the capture stream while a HIP graph is recorded
        t = r["sets"][r["i"] % len(r["sets"])]
        r["i"] += 1
        if r["fp8"]:
            self.W.w4a8_linear(r["lyr"].layer, r["M"], r["x"], r["xs"], t["qweight"], t["scales"], t["qzeros"],
                               t["perm"], None, r["y"], r["ws"], r["ws_b"], self.torch.cuda.current_stream())
            return
        self.W.w4a16_linear(r["lyr"].layer, r["M"], r["x"], t["qweight"], t["scales"], t["qzeros"], t["perm"], None,
                            r["y"], r["ws"] if r["ws_b"] else None, r["ws_b"], self.torch.cuda.current_stream())

    def per_case(self, runs):
        """Each case alone: a graph of back-to-back launches (rotating weight
        copies), the median of REPLAYS timed replays, per launch."""
        torch = self.torch
        out = []
        for r in runs:
            c, M = r["c"], r["M"]
            self.marker()
            for _ in range(3):
                self.launch(r)
            torch.cuda.synchronize()
            if self.args.reps:
                reps = self.args.reps
            else:
                est = self.timed(lambda n: [self.launch(r) for _ in range(n)], len(r["sets"]), 1) / len(r["sets"])
                # ~20 ms of launches per replay, at least one pass over the copies, at most 400
                reps = int(min(400, max(len(r["sets"]), 20.0 / max(est, 1e-4))))
            us = self.timed(lambda n: [self.launch(r) for _ in range(n)], reps, REPLAYS) * 1e3 / reps
            wb, tb = case_bytes(c, M)
            flops = 2.0 * M * c.K * c.N
            out.append(dict(K=c.K, N=c.N, M=M, kernel=r["kernel"], us=round(us, 3), reps=reps,
                            weight_GBps=round(wb / (us * 1e-6) / 1e9, 1),
                            total_GBps=round(tb / (us * 1e-6) / 1e9, 1),
                            TFLOPS=round(flops / (us * 1e-6) / 1e12, 2),
                            pct_hbm=round(100 * tb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                            pct_mfma=round(100 * flops / (us * 1e-6) / 1e12
                                           / (MFMA_F8_PEAK_TFLOPS if r["fp8"] else MFMA_F16_PEAK_TFLOPS), 1),
                            _wb=wb, _tb=tb, _flops=flops, _us=us))
        self.marker()
        return out

    def block(self, name, cases, runs, per_case, repack):
        c0 = cases[0]
        sum_us = sum(p["_us"] for p in per_case)
        wb = sum(p["_wb"] for p in per_case)
        fl = sum(p["_flops"] for p in per_case)
        fp8 = name == "w4a8"
        roof = roofline_of(per_case, MFMA_F8_PEAK_TFLOPS if fp8 else MFMA_F16_PEAK_TFLOPS)
        blk = {
            "workload": f"{name}: " + ", ".join(f"(K={c.K},N={c.N})" for c in cases)
                        + f" x M in {list(c0.Ms)}; {c0.fmt.upper()} "
                        + ("per-channel" if c0.group_size == -1 else f"g={c0.group_size}")
                        + (" zeros" if c0.has_zeros else " symmetric") + (" act-order" if c0.has_gidx else "")
                        + ("" if len({c.group_size for c in cases}) == 1 else " (+ per-channel variant)"),
            "act_dtype": c0.dtype,
            "compute_dtype": "fp8 e4m3 x int4 (static per-tensor activation scale)" if fp8 else c0.dtype,
            "cases": len(per_case),
            # each case once, back to back: packed-weight GB/s and flops of the set
            "weight_GBps": round(wb / (sum_us * 1e-6) / 1e9, 1),
            "TFLOPS": round(fl / (sum_us * 1e-6) / 1e12, 2),
            "sum_case_us": round(sum_us, 3),
            "roofline": roof,
            "per_case": [{k: v for k, v in p.items() if not k.startswith("_")} for p in per_case],
            "repack": repack,
        }
        return blk

    def workload(self, name):
        cases, runs, repack = self.setup(name)
        pc = self.per_case(runs)
        blk = self.block(name, cases, runs, pc, repack)
        if self.args.floor and name in FLOOR_WORKLOADS:
            blk["floor"] = self.floor(runs, pc)
        return cases, runs, pc, blk

    def floor(self, runs, per_case):
        """What a launch on the GEMM's grid can reach at this size: per case,
        a plain streaming read of the case's algorithmic bytes (rotated over
        buffers like the weights) and an empty kernel, both launched with the
        GEMM kernel's grid and workgroup size and timed like the GEMM (median
        of REPLAYS graph replays, per launch).  The streaming rate is the
        case's achievable target; gemm_frac_of_target = stream_us / gemm_us."""
        import ctypes
        torch, W = self.torch, self.W
        F = ctypes.CDLL(os.path.join(ROOT, "weight_only_int4_gptq_amd", "libw4floor.so"))
        F.w4floor_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32),
                                     ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        F.w4floor_empty.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_uint32, ctypes.c_int,
                                    ctypes.c_void_p]
        sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
        cases = []
        for tag, (r, p) in enumerate(zip(runs, per_case)):
            grid, threads = W.w4_launch_dims(r["lyr"].layer, r["M"])
            g = (ctypes.c_uint32 * 3)(*grid)
            nbytes = (p["_tb"] + 15) // 16 * 16
            R = max(2, math.ceil(ROTATE_BYTES / nbytes))
            bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda") for _ in range(R)]

            def stream(n, bufs=bufs, g=g, threads=threads, nbytes=nbytes, tag=tag):
                st = torch.cuda.current_stream().cuda_stream
                for i in range(n):
                    e = F.w4floor_stream(bufs[i % R].data_ptr(), nbytes, g, threads, sink.data_ptr(), tag % FLOOR_TAGS, st)
                    assert e == 0, f"w4floor_stream: hip error {e}"

            def empty(n, g=g, threads=threads, tag=tag):
                st = torch.cuda.current_stream().cuda_stream
                for _ in range(n):
                    e = F.w4floor_empty(g, threads, tag % FLOOR_TAGS, st)
                    assert e == 0, f"w4floor_empty: hip error {e}"

            stream(R)
            empty(1)
            torch.cuda.synchronize()
            reps = p["reps"]
            s_us = self.timed(stream, reps, REPLAYS) * 1e3 / reps
            e_us = self.timed(empty, reps, REPLAYS) * 1e3 / reps
            # the same bytes on other grids: the fastest plain streaming read found
            best = (s_us, list(grid), threads)
            for wgs in FLOOR_SWEEP_WGS:
                for th in FLOOR_SWEEP_THREADS:
                    g2 = (ctypes.c_uint32 * 3)(wgs, 1, 1)
                    us2 = self.timed(lambda n, g2=g2, th=th: stream(n, g=g2, threads=th), reps, REPLAYS) * 1e3 / reps
                    if us2 < best[0]:
                        best = (us2, [wgs, 1, 1], th)
            cases.append(dict(K=p["K"], N=p["N"], M=p["M"], kernel=p["kernel"], tag=tag % FLOOR_TAGS, grid=list(grid),
                              threads=threads, alg_bytes=p["_tb"], gemm_us=p["us"], stream_us=round(s_us, 3),
                              empty_us=round(e_us, 3),
                              target_GBps=round(p["_tb"] / (s_us * 1e-6) / 1e9, 1),
                              target_frac_of_peak=round(p["_tb"] / (s_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                              gemm_frac_of_target=round(s_us / p["_us"], 4),
                              best_stream_us=round(best[0], 3), best_stream_grid=best[1],
                              best_stream_threads=best[2],
                              best_stream_frac_of_peak=round(p["_tb"] / (best[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                              gemm_frac_of_best_stream=round(best[0] / p["_us"], 4)))
            del bufs
        tot_b = sum(c["alg_bytes"] for c in cases)
        tot_s = sum(c["stream_us"] for c in cases)
        tot_best = sum(c["best_stream_us"] for c in cases)
        tot_g = sum(c["gemm_us"] for c in cases)
        return {"what": "streaming read of each case's algorithmic bytes, and an empty kernel, on the GEMM's grid; "
                        "best_stream: the fastest streaming read of the same bytes over grids of "
                        f"{list(FLOOR_SWEEP_WGS)} workgroups x {list(FLOOR_SWEEP_THREADS)} threads and the GEMM's",
                "target_GBps": round(tot_b / (tot_s * 1e-6) / 1e9, 1),
                "best_stream_GBps": round(tot_b / (tot_best * 1e-6) / 1e9, 1),
                "gemm_GBps": round(tot_b / (tot_g * 1e-6) / 1e9, 1),
                "gemm_frac_of_target": round(tot_s / tot_g, 4),
                "gemm_frac_of_best_stream": round(tot_best / tot_g, 4),
                "per_case": cases}

    def steps(self, runs):
        """The timed steps of the headline: K passes over every case."""
        torch, args = self.torch, self.args
        for _ in range(args.warmup):
            for r in runs:
                self.launch(r)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ms = self.timed(lambda n: [self.launch(r) for _ in range(n) for r in runs], args.steps, 1) / args.steps
        return ms, time.perf_counter() - t0


def copy_probe(torch):
    """A plain device copy of known size (not timed): the reference that the
    HBM byte counters of a profiled run are scaled by."""
    src = torch.empty((COPY_PROBE_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_int4_gptq_amd as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    W.lib()
    if args.config == "moe":
        return main_moe(args, torch, W)
    B = Bench(args, torch, W)
    head = "decode" if args.config == "all" else args.config
    others = [w for w in WORKLOADS if w != head] if args.config == "all" else []

    cases, runs, per_case, blk = B.workload(head)
    copy_probe(torch)
    ms_step, wall = B.steps(runs)
    wbytes_step = sum(case_bytes(r["c"], r["M"])[0] for r in runs)
    flops_step = sum(2.0 * r["M"] * r["c"].K * r["c"].N for r in runs)
    value = wbytes_step / (ms_step * 1e-3) / 1e9
    unfused = {head: compare_unfused(torch, runs, per_case, B.stream)} if args.compare else None

    # headline roofline: the head workload's dominant bound
    roofs = blk["roofline"]
    roof = dict(max(roofs, key=lambda r: r["avg_launch_us"] * len(r["cases"])))
    if roof["bound"] == "hbm" and head == "decode" and not args.group_size:
        roof["traffic"] = measured_traffic()
    del runs
    torch.cuda.empty_cache()

    blocks = {head: blk}
    for w in others:
        cw, rw, pw, bw = B.workload(w)
        blocks[w] = bw
        if args.compare:
            unfused[w] = compare_unfused(torch, rw, pw, B.stream)
        del rw
        torch.cuda.empty_cache()

    cpu = None if args.no_cpu else cpu_baseline(cases, args.cpu_seconds)
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
            "workload": blk["workload"],
            "cases": len(per_case), "act_dtype": c0.dtype, "weight_rotation_MiB": ROTATE_BYTES >> 20,
            "copy_probe_MiB": COPY_PROBE_BYTES >> 20,
        },
        "timing": ("eager launches" if args.eager else
                   "HIP graph of the K timed steps (one untimed replay uploads it, one replay is timed); "
                   f"per case: median of {REPLAYS} replays of a graph of back-to-back launches"),
        "tflops_step": round(flops_step / (ms_step * 1e-3) / 1e12, 3),
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": blocks,
        "dequant_then_gemm": unfused,
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
    B = Bench(args, torch, W)
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

    wbytes = E * K * N // 2
    per_case = []
    for r in runs:
        B.marker()
        for _ in range(3):
            launch(r)
        torch.cuda.synchronize()
        reps = 20 if r["rows"] >= 1024 else 60
        us = B.timed(lambda n: [launch(r) for _ in range(n)], reps, REPLAYS) * 1e3 / reps
        tb = wbytes + E * G * N * 2 + E * G * N // 2 + r["rows"] * (K + N) * 2
        fl = 2.0 * r["rows"] * K * N
        per_case.append(dict(K=K, N=N, M=r["rows"], tokens=r["T"], rows_per_expert=r["counts"],
                             kernel="w4a16_moe_linear", us=round(us, 3),
                             weight_GBps=round(wbytes / (us * 1e-6) / 1e9, 1),
                             TFLOPS=round(fl / (us * 1e-6) / 1e12, 2), _tb=tb, _flops=fl, _us=us))
    B.marker()

    for _ in range(args.warmup):
        for r in runs:
            launch(r)
    torch.cuda.synchronize()
    t0w = time.perf_counter()
    ms_step = B.timed(lambda n: [launch(r) for _ in range(n) for r in runs], args.steps, 1) / args.steps
    wall = time.perf_counter() - t0w
    value = len(runs) * wbytes / (ms_step * 1e-3) / 1e9
    roofs = roofline_of(per_case)
    cpu = None
    if not args.no_cpu:
        import oracle as O
        xs = normal_acts(seeded(9, 4, K), (4, K), "fp16")
        tc = time.perf_counter()
        O.reference_moe(xs, np.array([0, 4]), "awq", "fp16", [experts[0]], 128)
        dt = time.perf_counter() - tc
        cpu = {"value": round((K * N // 2) / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
               "kind": "oracle", "sample": "one expert (K=4096, N=28672) on 4 rows", "seconds": round(dt, 2)}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded uniform int4 codes/zeros, uniform scales, N(0,1) activations, random top-2 routing)",
        "config": {"workload": f"moe: E={E} experts of (K={K},N={N}) AWQ g=128 zeros, top-{MOE_TOPK} routing of "
                               f"{list(MOE_TOKENS)} tokens", "cases": len(runs), "act_dtype": "fp16",
                   "weight_rotation_MiB": ROTATE_BYTES >> 20},
        "timing": f"HIP graph of the timed launches; per case: median of {REPLAYS} replays",
        "wall_s_timed": round(wall, 3), "roofline": roofs[-1], "roofline_all": roofs, "cpu_baseline": cpu,
        "per_case": [{k: v for k, v in p.items() if not k.startswith("_")} for p in per_case],
    }
    print(json.dumps(out), flush=True)


def compare_unfused(torch, runs, per_case, stream):
    """The unfused path the pages describe for large batches: the library's
    dense dequantization kernel writes W [K, N] in the activation dtype, then
    torch.matmul (the vendor GEMM) computes x W.  Each part is timed with HIP
    events over back-to-back direct launches, per case, next to the fused
    kernel's time from the per-case timing."""
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


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(cases, seconds):
    """The CPU oracle, as it stands, on a bounded sample of the headline
    workload: for each (layer, M) case in order, until ``seconds`` of CPU time
    are spent, the oracle's three phases are timed separately:
      1. unpack + AWQ order fix + standard repack (awq_to_std, then the
         standard unpack to codes; NumPy integer ops, one thread),
      2. float64 dequantization per group (one thread),
      3. float64 matmul (BLAS dgemm on the BLAS threads).
    ``value`` is packed-weight GB/s over the three phases together, in the
    metric's unit."""
    import oracle as O
    from synthetic import make_acts, make_layer_inputs
    ph = {"unpack_repack_s": 0.0, "dequant_s": 0.0, "matmul_s": 0.0}
    done, wbytes = [], 0
    spent = 0.0
    for _ in range(8):  # passes over the workload until `seconds` of CPU time are spent
        for c in cases:
            Lw = make_layer_inputs(c)
            for M in c.Ms:
                x = make_acts(c, M)
                t0 = time.perf_counter()
                if c.fmt == "awq":
                    sw, sz = O.awq_to_std(Lw["qweight"], Lw["qzeros"])
                else:
                    sw, sz = Lw["qweight"], Lw["qzeros"]
                q = O.unpack_std(sw)
                z = None if sz is None else O.unpack_std_zeros(sz)
                t1 = time.perf_counter()
                Wd = O.dequant(q, z, O.act_to_f64(Lw["scales"], c.dtype),
                               O.group_index(c.K, c.group_size, Lw["g_idx"]))
                t2 = time.perf_counter()
                O.linear_ref(O.act_to_f64(x, c.dtype), Wd)
                t3 = time.perf_counter()
                ph["unpack_repack_s"] += t1 - t0
                ph["dequant_s"] += t2 - t1
                ph["matmul_s"] += t3 - t2
                spent += t3 - t0
                wbytes += c.K * c.N // 2
                done.append(f"(K={c.K},N={c.N},M={M})")
                del Wd, q
                if spent >= seconds:
                    break
            if spent >= seconds:
                break
        if spent >= seconds:
            break
    return {"value": round(wbytes / spent / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "phases": {k: round(v, 3) for k, v in ph.items()},
            "phase_threads": {"unpack_repack": 1, "dequant": 1, "matmul": blas_threads()},
            "sample": f"{len(done)} oracle layer calls cycling through the decode cases "
                      + " ".join(dict.fromkeys(done)), "seconds": round(spent, 2)}


if __name__ == "__main__":
    main()
