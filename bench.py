#!/usr/bin/env python3
"""Benchmark of the W4A16 GEMM on one MI355X; prints one JSON line.

Default workload (the decode configuration of the headline metric): one step
is two GEMMs, M = 1 and M = 5, K = 5120, N = 17408, bf16 activations, uint4
weights with group size 128, symmetric. ``value`` is the effective HBM
bandwidth of the step: algorithmic bytes (packed weights + scales + zero
points + activations + output) over the step's wall time on the GPU. Weight
sets are rotated over at least 512 MB of distinct copies so that the 256 MB
Infinity Cache cannot hold them between launches; inputs are resident in HBM
before timing starts.

``--workload NAME`` times one of the other workloads instead (prefill reports
TFLOP/s); ``--all`` prints one line per workload. The prefill GEMM (M = 2048)
is always timed too and reported under ``extra``.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2516.6      # MI355X dense fp16/bf16 (256 CU x 4096 flop/clk x 2.4 GHz)
ROTATE_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    help="decode (M=1 and M=5), prefill, k2112, tiny, sweep_m<M>, sweep_pc16")
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill-extra", action="store_true")
    ap.add_argument("--warm", action="store_true", help="no weight rotation (cache-warm)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    ap.add_argument("--kpacked", action="store_true",
                    help="time the workload with the weights K-packed ([N, K/8], w4a16_gemm_kpacked)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context ceilings (plain streaming read, dense bf16 matmul)")
    ap.add_argument("--read-probe", type=int, default=0, metavar="BYTES",
                    help="only time the plain streaming read of BYTES (context ceiling) and exit")
    ap.add_argument("--issue-probe", action="store_true",
                    help="only run the instruction-issue probe (cycles per instruction of one "
                         "wavefront, MFMA with 0-32 FMAs each, 1 and 2 wavefronts per SIMD) and exit")
    ap.add_argument("--prefill-stages", default="",
                    help="comma-separated 64-row K stages per split (0 = selector's) to force on "
                         "the prefill route for --workload; one line per value (split-count sweep)")
    return ap.parse_args()


def alg_bytes(w, kpacked: bool = False) -> int:
    """Packed weights + scales + zero points (packed 8 per int32, or one byte
    each in the K-packed layout) + activations + output."""
    ng = w.K // w.group_size
    zp = (ng * w.N if kpacked else ng * (w.N // 8) * 4) if w.has_zp else 0
    return w.K * w.N // 2 + ng * w.N * 2 + zp + w.M * w.K * 2 + w.M * w.N * 2


def flops(w) -> int:
    return 2 * w.M * w.N * w.K


class Launch:
    """Device-resident inputs of one workload with rotated weight copies.

    Calls go straight to the C ABI (``w4a16_gemm_ws`` with one caller-owned
    workspace, or ``w4a16_gemm_kpacked``) with argument tuples built once per
    copy, so the host enqueues faster than the GPU drains.
    """

    def __init__(self, w, torch, W, synthetic, rotate: bool, kpacked: bool = False):
        d = synthetic.draw_workload(w)
        dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
        dev = torch.device("cuda", 0)
        self.w = w
        self.torch = torch
        self.kpacked = kpacked
        self.a = torch.from_numpy(d["a_bits"].view("int16")).view(dt).to(dev)
        if kpacked:
            # the same weights K-packed: [N, K/8] in ExLlama order, scales and
            # zero points [N, K/G] (zero points one byte each)
            bq = torch.from_numpy(W.pack_int4_kshuffle(np.ascontiguousarray(d["q"].T))).to(dev)
            s = torch.from_numpy(np.ascontiguousarray(d["s_bits"].T).view("int16")).view(dt).to(dev)
            qz = None if d["z"] is None else torch.from_numpy(np.ascontiguousarray(d["z"].T)).to(dev)
        else:
            bq = torch.from_numpy(W.pack_int4(d["q"])).to(dev)
            s = torch.from_numpy(d["s_bits"].view("int16")).view(dt).to(dev)
            qz = None if d["z"] is None else torch.from_numpy(W.pack_int4(d["z"])).to(dev)
        weight_bytes = bq.numel() * 4 + s.numel() * 2 + (0 if qz is None else qz.numel() * qz.element_size())
        copies = max(1, math.ceil(ROTATE_BYTES / weight_bytes)) if rotate else 1
        self.sets = [(bq, s, qz)] + [(bq.clone(), s.clone(), None if qz is None else qz.clone())
                                     for _ in range(copies - 1)]
        self.out = torch.empty((w.M, w.N), dtype=dt, device=dev)
        # caller-owned scratch (counter region zeroed once), shared by the
        # rotated copies: the launches run one after another on one stream
        nb = 0 if kpacked else W.workspace_bytes(w.M, w.K, w.N, w.group_size, dt,
                                                 torch.cuda.get_device_properties(0).multi_processor_count)
        self.ws = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb else None
        self.W = W
        self.args = None
        self.i = 0

    def bind(self):
        """Argument tuples for the current stream (call again inside a capture)."""
        if self.kpacked:
            self.args = [self.W.gemm_kpacked_args(self.a, bq, s, qz, self.w.group_size, 8, self.out)
                         for bq, s, qz in self.sets]
        else:
            self.args = [self.W.gemm_ws_args(self.a, bq, s, qz, self.w.group_size, 8, self.out,
                                             self.ws) for bq, s, qz in self.sets]

    def __call__(self):
        if self.kpacked:
            self.W.launch_kpacked(self.args[self.i % len(self.args)])
        else:
            self.W.launch_ws(self.args[self.i % len(self.args)])
        self.i += 1


def time_launches(launches, steps, warmup, torch):
    """Eager: per-launch durations from HIP events on the launch stream, and
    the wall time of the timed steps (synchronised on both sides)."""
    stream = torch.cuda.current_stream()
    for L in launches:
        L.bind()
    for _ in range(warmup):
        for L in launches:
            L()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(steps):
        for j, L in enumerate(launches):
            ev[k][j][0].record(stream)
            L()
            ev[k][j][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per = [[ev[k][j][0].elapsed_time(ev[k][j][1]) for k in range(steps)]
           for j in range(len(launches))]
    return total_ms, per


def time_graph(launches, steps, torch):
    """The same K steps captured once into a HIP graph and replayed: no host
    work between kernels. Returns the wall time of one replay."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for L in launches:
                L.bind()
            for _ in range(steps):
                for L in launches:
                    L()
    torch.cuda.synchronize()
    for _ in range(3):              # untimed warm replays (clocks settle)
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    for L in launches:              # back to the eager stream
        L.bind()
    return t0.elapsed_time(t1)


def _graph_time(fn_list, torch):
    """Capture one call of each fn into a HIP graph, replay it three times
    untimed, then once timed with HIP events on the replaying stream;
    returns ms per call."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for f in fn_list:
                f()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / len(fn_list)


def context_read(torch, nbytes, launches=60):
    """Achievable HBM read rate of one launch of ``nbytes``: a plain
    streaming-read kernel (``libw4a16_probe.so``) over copies rotated across
    >= 512 MB, graph-replayed; the best of a few grid sizes."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "weight_only_int4_unpack_amd", "libw4a16_probe.so"))
    probe.w4a16_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = (nbytes + 15) // 16 * 16
    copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
    bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
            for _ in range(copies)]
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        out = torch.empty(blocks, dtype=torch.int32, device="cuda")

        def mk(b, blocks=blocks, out=out):
            def f():
                st = probe.w4a16_probe_read(b.data_ptr(), nbytes, blocks, 0x9E3779B9,
                                            out.data_ptr(), torch.cuda.current_stream().cuda_stream)
                assert st == 0, st
            return f
        ms = _graph_time([mk(bufs[i % copies]) for i in range(launches)], torch)
        if best is None or ms < best[0]:
            best = (ms, blocks)
    ms, blocks = best
    del bufs
    return {"bytes": nbytes, "us_per_launch": round(ms * 1e3, 2),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "workgroups": blocks,
            "how": f"plain 16-byte streaming read, {copies} copies rotated, {launches} launches "
                   "graph-replayed, best grid of 1024/2048/4096/8192 x 256 threads"}


def context_matmul(torch, M=2048, K=5120, N=17408, launches=20):
    """Dense bf16 torch.matmul (hipBLASLt) at the prefill shape, the weights
    as a plain [K, N] bf16 matrix rotated over >= 512 MB, graph-replayed."""
    a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    copies = max(2, math.ceil(ROTATE_BYTES / (K * N * 2)))
    ws = [torch.randn(K, N, device="cuda").to(torch.bfloat16) for _ in range(copies)]
    out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    for w in ws:                                     # warm up the library's choice
        torch.matmul(a, w, out=out)
    torch.cuda.synchronize()
    fns = [(lambda w=ws[i % copies]: torch.matmul(a, w, out=out)) for i in range(launches)]
    ms = _graph_time(fns, torch)
    del ws
    tf = 2 * M * N * K / (ms * 1e-3) / 1e12
    return {"shape": [M, K, N], "us_per_launch": round(ms * 1e3, 2), "tflops": round(tf, 1),
            "frac_of_mfma_peak": round(tf / MFMA_PEAK_TFLOPS, 4),
            "how": f"torch.matmul bf16 [M,K] x [K,N], {copies} weight copies rotated, "
                   f"{launches} launches graph-replayed"}


def plan_time(w, pl, torch, W, synthetic, launches=40):
    """Graph-replayed per-launch time of workload w with plan pl
    (w4a16_gemm_planned; the library's workspace of the capturing stream is
    made by one uncaptured call first)."""
    L = Launch(w, torch, W, synthetic, rotate=True)
    run = lambda i: W.gemm(L.a, *L.sets[i % len(L.sets)][:2], L.sets[i % len(L.sets)][2],
                           w.group_size, 8, out=L.out, plan=pl)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(launches):
                run(i)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    return round(t0.elapsed_time(t1) * 1e3 / launches, 2)


def forced_prefill(name, stages, torch, W, synthetic):
    """One workload on the prefill route with the K stages per split forced."""
    w = synthetic.WORKLOADS[name]
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    pl = W.plan(w.M, w.K, w.N, w.group_size, w.has_zp, dt, route=W.ROUTE_PREFILL,
                steps_per_wave=stages)
    return {"workload": name, "stages_per_split": pl.steps_per_wave, "splits": pl.splits,
            "workgroups": pl.grid, "us_per_launch": plan_time(w, pl, torch, W, synthetic)}


def issue_probe(torch, iters=4000):
    """Shader-clock cycles per loop trip of probe_issue_kernel: eight MFMA
    chains with NV FMAs after each MFMA, or 64 FMAs alone; 256 workgroups
    with 100 KB of LDS (one per CU: one wavefront per SIMD) or 512 with 60 KB
    (two per SIMD). Reports cycles per issued instruction of one wavefront
    (the loop's instruction count is read from the build's own assembly and
    given in the output's note)."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "weight_only_int4_unpack_amd", "libw4a16_probe.so"))
    probe.w4a16_probe_issue.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3
    out = torch.empty(512 * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(1, dtype=torch.int64, device="cuda")
    res = []
    for per_simd, blocks, lds in ((1, 256, 100 * 1024), (2, 512, 60 * 1024)):
        for nv in (0, 8, 16, 32, -1):
            for _ in range(5):
                st = probe.w4a16_probe_issue(nv, blocks, lds, iters, out.data_ptr(), clk.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream)
                assert st == 0, st
            torch.cuda.synchronize()
            cyc = clk.item() / iters
            res.append({"wavefronts_per_simd": per_simd,
                        "loop": "64 FMAs" if nv < 0 else f"8 MFMAs + {nv} FMAs each",
                        "cycles_per_trip": round(cyc, 1)})
    return res


def load_traffic(path, name, src_hash):
    """HBM bytes per launch of this workload, from rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes (scaled by a plain-copy calibration), or None when the
    record is missing or was taken on another version of the kernels."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(name)
    if not rec or rec.get("kernel_sha") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(workloads, budget_s=12.0):
    """The oracle (untuned) on the host, on a bounded sample of the workload."""
    import numpy as np
    import oracle as O
    from weight_only_int4_unpack_amd import synthetic
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    inputs = []
    for w in workloads:
        d = synthetic.draw_workload(w)
        inputs.append((w, d["a_bits"], O.pack_int4(d["q"]), d["s_bits"],
                       None if d["z"] is None else O.pack_int4(d["z"])))
    done_bytes = 0
    calls = 0
    t0 = time.perf_counter()
    while True:
        for w, a, bq, s, qz in inputs:
            O.gemm(a, bq, s, qz, w.group_size, 8, w.dtype)
            done_bytes += alg_bytes(w)
            calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done_bytes / el / 1e12, "unit": "TB/s", "cores": blas, "kind": "oracle",
            "sample": f"{calls} full oracle GEMMs ({'+'.join(w.name for w in workloads)}) in "
                      f"{el:.1f} s: NumPy unpack/dequant on one thread, fp32 matmul on "
                      f"{blas} OpenBLAS threads; host has {os.cpu_count()} CPUs, affinity "
                      f"{len(os.sched_getaffinity(0))}"}


def run_workload(names, steps, warmup, rotate, torch, W, synthetic, graph=True, kpacked=False):
    ws = [synthetic.WORKLOADS[n] for n in names]
    launches = [Launch(w, torch, W, synthetic, rotate, kpacked) for w in ws]
    total_ms, per = time_launches(launches, steps, warmup, torch)
    graph_ms = time_graph(launches, steps, torch) if graph else None
    res = []
    for w, d in zip(ws, per):
        d = sorted(d)
        res.append({"name": w.name, "median_us": 1e3 * d[len(d) // 2],
                    "mean_us": 1e3 * sum(d) / len(d), "bytes": alg_bytes(w, kpacked),
                    "flops": flops(w),
                    "plan": W.plan(w.M, w.K, w.N, w.group_size, w.has_zp,
                                   torch.float16 if w.dtype == "fp16" else torch.bfloat16).as_dict()})
    return total_ms, graph_ms, res


def kernel_source_hash() -> str:
    import hashlib
    src = os.path.join(ROOT, "weight_only_int4_unpack_amd", "csrc", "w4a16_kernels.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this build "
              "runs the GEMM on a single MI355X (sharding is described, not built).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from weight_only_int4_unpack_amd import synthetic
    from weight_only_int4_unpack_amd import w4a16 as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    rotate = not args.warm
    if args.read_probe:
        print(json.dumps({"read_probe": context_read(torch, args.read_probe)}), flush=True)
        return
    if args.issue_probe:
        for r in issue_probe(torch):
            print(json.dumps({"issue_probe": r}), flush=True)
        return
    if args.prefill_stages:
        for st in (int(x) for x in args.prefill_stages.split(",")):
            print(json.dumps({"forced_prefill": forced_prefill(args.workload, st, torch, W,
                                                               synthetic)}), flush=True)
        return

    if args.copy_probe:
        x = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(4):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    groups = {"decode": ["decode_m1", "decode_m5"]}
    todo = ([["decode_m1", "decode_m5"], ["prefill"], ["k2112"], ["tiny"], ["sweep_pc16"]]
            + [[f"sweep_m{m}"] for m in (1, 2, 4, 5, 6, 16, 64, 256, 4096)]) if args.all \
        else [groups.get(args.workload, [args.workload])]
    # --all also times the K-packed layout ([N, K/8], w4a16_gemm_kpacked) on
    # the decode-sized workloads
    todo = [(n, args.kpacked) for n in todo] + ([(n, True) for n in (
        ["decode_m1", "decode_m5"], ["k2112"], ["tiny"], ["sweep_pc16"], ["sweep_m1"], ["sweep_m5"],
        ["sweep_m16"])] if args.all else [])

    cpu = None
    for names, kpacked in todo:
        wl = [synthetic.WORKLOADS[n] for n in names]
        is_prefill = any(w.M > 16 for w in wl)
        steps = args.steps if not is_prefill else max(5, min(args.steps, 50))
        eager_ms, graph_ms, res = run_workload(names, steps, args.warmup, rotate, torch, W,
                                               synthetic, kpacked=kpacked)
        n_launch = len(res)
        step_bytes = sum(r["bytes"] for r in res)
        step_flops = sum(r["flops"] for r in res)
        # timed region: the K steps replayed from one HIP graph (no host work
        # between kernels), bracketed by synchronisation; HIP events on the
        # launch stream give its duration
        ms_per_step = graph_ms / steps
        launch_us = 1e3 * ms_per_step / n_launch
        if is_prefill:
            metric = "W4A16 GEMM TFLOP/s (prefill, MFMA path), 1 MI355X"
            value = step_flops / (ms_per_step * 1e-3) / 1e12
            unit = "TFLOP/s"
            ach = step_flops / n_launch / (launch_us * 1e-6) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4)}
        else:
            metric = "W4A16 GEMM effective HBM TB/s (decode M<=8), 1 MI355X"
            value = step_bytes / (ms_per_step * 1e-3) / 1e12
            unit = "TB/s"
            ach = step_bytes / n_launch / (launch_us * 1e-6) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
        roof["traffic"] = None if kpacked else load_traffic(args.traffic, "+".join(names),
                                                             kernel_source_hash())
        line = {
            "metric": metric, "value": round(value, 4), "unit": unit, "n_gpus": 1,
            "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": wl[0].dtype, "data": "synthetic",
            "config": {"workload": "+".join(names),
                       "shapes": [{"M": w.M, "K": w.K, "N": w.N, "group_size": w.group_size,
                                   "zero_points": w.has_zp} for w in wl],
                       "weights_rotated_over_mb": 0 if not rotate else ROTATE_BYTES >> 20,
                       "launch": "K steps captured in one HIP graph, replayed once",
                       "layout": "[N, K/8] K-packed" if kpacked else "[K, N/8]",
                       "parallelism": "single GPU"},
            "roofline": roof,
            "eager": {"ms_per_step": round(eager_ms / steps, 5),
                      "how": "same steps launched one by one through the C ABI",
                      "launches": res},
        }
        if kpacked:
            line["metric"] = line["metric"].replace("W4A16 GEMM", "W4A16 GEMM, K-packed weights,")
            for r in res:
                r["plan"] = {"kernel": "kpacked", "block": "16 columns x 16 rows, all of K"}
        if names == ["decode_m1", "decode_m5"] and not kpacked and not args.no_prefill_extra:
            # 20 graph-replayed steps after 10 warm-up launches (the first
            # launches of a fresh process run measurably slower)
            _, pg, pres = run_workload(["prefill"], 20, 10, rotate, torch, W, synthetic)
            pf = pres[0]
            pus = 1e3 * pg / 20
            tf = pf["flops"] / (pus * 1e-6) / 1e12
            line["extra"] = {"prefill": {"tflops": round(tf, 1),
                                         "frac_of_mfma_peak": round(tf / MFMA_PEAK_TFLOPS, 4),
                                         "us_per_launch": round(pus, 2),
                                         "plan": pf["plan"]}}
        if names == ["decode_m1", "decode_m5"] and not kpacked and not args.no_context:
            # achievable ceilings on this GPU, for reading value and the
            # prefill figure against (context, not the specification peaks)
            ctx = {"read_46mb": context_read(torch, res[0]["bytes"])}
            if not args.no_prefill_extra:
                ctx["dense_bf16_matmul_prefill_shape"] = context_matmul(torch)
            line.setdefault("extra", {})["context"] = ctx
        if not args.no_cpu and cpu is None and not args.all:
            cpu = cpu_baseline(wl)
            if is_prefill:
                cpu["sample"] += " (value in TB/s of algorithmic bytes)"
        line["cpu_baseline"] = cpu
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
