#!/usr/bin/env python3
"""Benchmark of the decode hot path on one MI355X: activation FP4 quantisation
followed by the fused NVFP4 + binary low-rank product (libbiloco_hip).

One step = biloco_gemm_lowrank_quant (the activation's FP4 quantisation and
the fused product) on one batch of seeded synthetic decode inputs (weights
resident in HBM).  K steps are captured in a
HIP graph, each on a different copy of the weights (R codes, R scales, U, V)
so that together they span >= 1.2 GB and the 256 MB Infinity Cache cannot
serve them; the timed region replays the graph once between synchronisations.

Prints ONE JSON line (see the keys below).  --gpus must be 1.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 10^9 B/s
ROT_BYTES = 1.2e9              # distinct weight bytes a timed graph walks through
SCHED_NAMES = {1: "unfused", 2: "fused_gemv", 3: "fused_mfma", 4: "composed",
               5: "composed_mfma", 6: "mfma_allwg", 7: "mfma_side", 8: "mfma_zepi"}
METRIC = "fused GEMM µs/call + effective HBM GB/s (% peak) at M=1..32, r=512"


def algorithmic_bytes(M: int, N: int, K: int, r: int) -> int:
    """Bytes one product call must move once: R codes + R scales + g + the FP4
    activation (codes + scales) + x (when r > 0) + U + V + alpha + y."""
    W = (r + 31) // 32
    b = N * K // 2 + N * K // 16 + 4 + M * K // 2 + M * K // 16 + 2 * M * N
    if r > 0:
        b += 2 * M * K + 4 * W * (N + K) + 2 * r
    return b


def code_text(src: str) -> str:
    """C/C++/HIP source without its comments and with runs of whitespace
    collapsed: what the compiler sees, so that an edit of a comment leaves
    the hash of the kernels alone."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":                            # string or character literal
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


# the launches of one product call per default schedule; the roofline divides
# the call's algorithmic bytes by the call's time, which the kernel trace
# gives as the sum of these kernels' averages
CALL_KERNELS = {"unfused": "z_kernel + fused_gemv_kernel",
                "fused_mfma": "mfma_z_kernel + mfma_zreduce_kernel (K > 7168) + "
                              "mfma_product_kernel + mfma_epilogue_kernel (split K)",
                "mfma_zepi": "mfma_product_kernel (z in its side workgroups) + mfma_epilogue_zc_kernel"}


# the sources a schedule's launches are built from (the hash that keys its
# counter records); other schedules' files may change without voiding them
SCHED_FILES = {"fused_gemv": ["k_fused_gemv.hip", "biloco_device.h", "biloco_internal.h"],
               "mfma_allwg": ["k_fused_mfma.hip", "biloco_device.h", "biloco_internal.h"],
               "mfma_side": ["k_fused_mfma.hip", "biloco_device.h", "biloco_internal.h"],
               "unfused": ["k_fused_gemv.hip", "biloco_device.h", "biloco_internal.h"],
               "fused_mfma": ["k_fused_mfma.hip", "biloco_device.h", "biloco_internal.h"],
               "mfma_zepi": ["k_fused_mfma.hip", "biloco_device.h", "biloco_internal.h"]}


def source_hash(sched_name: str | None = None) -> str:
    """Hash of the kernel sources' code (comments excluded): all of csrc/, or
    only the files of one schedule's kernels."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "bit_weight_gemm_amd", "csrc", "*")))
    if sched_name in SCHED_FILES:
        files = [f for f in files if os.path.basename(f) in SCHED_FILES[sched_name]]
    for f in files:
        with open(f, "r", encoding="utf-8") as fh:
            h.update(os.path.basename(f).encode())
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg: int, sched_name: str):
    """HBM bytes per call from the committed rocprofv3 --pmc summary, if it was
    taken on the current sources of the schedule's kernels; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{sched_name}_config{cfg}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(sched_name):
        return None
    return d.get("bytes_per_call")


class Rotation:
    """B device copies of the weight operands of one problem."""

    def __init__(self, prob, n_sets: int):
        import torch
        self.n = n_sets
        self.wc = [prob.w_codes] + [prob.w_codes.clone() for _ in range(n_sets - 1)]
        self.ws = [prob.w_scales] + [prob.w_scales.clone() for _ in range(n_sets - 1)]
        if prob.r > 0:
            self.up = [prob.u_packed] + [prob.u_packed.clone() for _ in range(n_sets - 1)]
            self.vp = [prob.v_packed] + [prob.v_packed.clone() for _ in range(n_sets - 1)]
        else:
            self.up = self.vp = [None] * n_sets
        torch.cuda.synchronize()

    def kw(self, i: int) -> dict:
        j = i % self.n
        return dict(w_codes=self.wc[j], w_scales=self.ws[j], u_packed=self.up[j],
                    v_packed=self.vp[j])


def weight_bytes(prob) -> int:
    b = prob.w_codes.numel() + prob.w_scales.numel()
    if prob.r > 0:
        b += 4 * (prob.u_packed.numel() + prob.v_packed.numel())
    return b


def time_graph(fn_step, n: int, reps: int = 3):
    """Capture n calls of fn_step(i) in a HIP graph; return (best GPU seconds
    per call over reps replays, graph)."""
    import torch
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for i in range(n):
            fn_step(i, st)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3 / n)
    return best, g


def gemm_call_time(prob, sched: int, rot: Rotation | None, calls: int) -> float:
    def step(i, st):
        kw = rot.kw(i) if rot is not None else {}
        prob.gemm(sched, stream=st, **kw)
    t, _ = time_graph(step, calls)
    return t


def weight_quant_table() -> dict:
    """biloco_quant_weight_nvfp4 on fp32 residuals of the decode weight shapes:
    time per call (a graph of 20 calls over 4 copies of the matrix, 420+ MB),
    and algorithmic bytes (read w once, write codes and scales) per second."""
    import torch
    from bit_weight_gemm_amd import binding as B
    from bit_weight_gemm_amd import workloads as wl
    res = {}
    for N, K in ((5120, 5120), (13824, 5120)):
        w0 = torch.from_numpy(wl.make_residual(N, K, seed=N + K, outliers=True)).cuda()
        ws = [w0] + [w0.clone() for _ in range(3)]
        c = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
        g = torch.empty(4, dtype=torch.float32, device="cuda")[:1]
        wsp = torch.empty(B.biloco_quant_weight_workspace_bytes(N, K), dtype=torch.uint8,
                          device="cuda")
        for i in range(4):
            B.biloco_quant_weight_nvfp4(ws[i], c, s, g, wsp)
        torch.cuda.synchronize()
        t, _ = time_graph(lambda i, st: B.biloco_quant_weight_nvfp4(ws[i % 4], c, s, g, wsp,
                                                                    stream=st), 20)
        alg = N * K * 4 + N * K // 2 + N * K // 16 + 4
        res[f"{N}x{K}"] = {"us_per_call": round(t * 1e6, 2), "GBps": round(alg / t / 1e9, 1),
                           "pct_peak": round(100 * alg / t / 1e9 / PEAK_HBM_GBS, 2),
                           "bytes_per_call": alg, "passes_over_w": 2}
        del ws, w0, c, s
        torch.cuda.empty_cache()
    return res


def decompose_time(m: int = 5120, n: int = 5120, r: int = 512, T: int = 5) -> dict:
    """biloco_peel_decompose on a seeded fp32 5120 x 5120 weight: one
    full decomposition (r terms of T sign steps, refit, residual) between HIP
    events on torch's stream, after one untimed run.  Each sign step is one
    pass over W for R v and one for R^T u; the residual reads W and writes R:
    (2 T r + 2) * 4 m n bytes in all."""
    import numpy as np
    import torch
    from bit_weight_gemm_amd import binding as B
    from bit_weight_gemm_amd import workloads as wl
    W = torch.from_numpy(wl.make_residual(m, n, seed=2024, outliers=True)).cuda()
    vi = torch.from_numpy(wl.make_start_signs(r, n, seed=77).view(np.int32)).cuda()
    ws = torch.empty(B.biloco_peel_workspace_bytes(m, n, r), dtype=torch.uint8, device="cuda")
    B.biloco_peel_decompose(W, r, T, vi, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    B.biloco_peel_decompose(W, r, T, vi, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    nbytes = (2 * T * r + 2) * 4 * m * n
    return {"m": m, "n": n, "r": r, "T": T, "ms": round(t * 1e3, 2),
            "GBps": round(nbytes / t / 1e9, 1),
            "pct_peak": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 2),
            "bytes": nbytes,
            "note": f"W is {4 * m * n / 1e6:.0f} MB, which the 256 MB Infinity Cache holds: most of "
                    "its passes are served from that cache, so pct_peak is a rate against the HBM "
                    "peak, not an HBM measurement"}


def stream_floor(configs=(1, 2, 3, 4), calls: int = 200) -> dict:
    """The floors a product call is compared with, in the same graph-replay
    form the product is timed in: one launch that only reads the config's
    algorithmic byte count from HBM (a plain 16-byte-per-lane read kernel,
    buffers rotated over >= 1.2 GB so that the Infinity Cache cannot serve
    them), and one empty launch."""
    import ctypes
    import math
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_weight_gemm_amd", "libbiloco_floor.so"))
    lib.biloco_floor_read.restype = ctypes.c_int
    lib.biloco_floor_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p]
    lib.biloco_floor_empty.restype = ctypes.c_int
    lib.biloco_floor_empty.argtypes = [ctypes.c_void_p]
    from bit_weight_gemm_amd import workloads as wl
    out = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    res = {}
    for c in configs:
        cf = wl.CONFIGS[c]
        nb = algorithmic_bytes(cf["M"], cf["N"], cf["K"], cf["r"])
        n_sets = max(2, math.ceil(ROT_BYTES / nb))
        bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(n_sets)]
        torch.cuda.synchronize()

        def step(i, st, bufs=bufs, nb=nb):
            assert lib.biloco_floor_read(bufs[i % len(bufs)].data_ptr(), nb, out.data_ptr(), 256,
                                         st.cuda_stream) == 0
        t, _ = time_graph(step, calls)
        res[f"config{c}"] = {"bytes": nb, "us_per_call": round(t * 1e6, 3),
                             "GBps": round(nb / t / 1e9, 1),
                             "pct_peak": round(100 * nb / t / 1e9 / PEAK_HBM_GBS, 2)}
        del bufs
        torch.cuda.empty_cache()
    t, _ = time_graph(lambda i, st: lib.biloco_floor_empty(st.cuda_stream), calls)
    res["empty_launch_us"] = round(t * 1e6, 3)
    return res


def cpu_baseline(cfg: int, seconds: float):
    import numpy as np
    import oracle
    from bit_weight_gemm_amd import workloads as wl
    d = wl.make_config(cfg)
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.quant_act_fp4(d["x"])
        oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"], d["alpha"])
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    nb = algorithmic_bytes(d["M"], d["N"], d["K"], d["r"])
    res = {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
           "kind": "oracle", "us_per_call": round(dt * 1e6, 1),
           "sample": f"{n} full calls of the config-{cfg} product on the host (quantise x, then "
                     f"y in fp64 over all M*N outputs), same seeded inputs as the GPU"}
    # the same on one thread (a bounded sample: whole calls for about a
    # fifth of the time above)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    n1, t1 = 0, time.perf_counter()
    while True:
        oracle.quant_act_fp4(d["x"])
        oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"], d["alpha"])
        n1 += 1
        if time.perf_counter() - t1 >= seconds / 5:
            break
    oracle.set_num_threads(threads)
    dt1 = (time.perf_counter() - t1) / n1
    res["one_thread"] = {"value": round(nb / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "us_per_call": round(dt1 * 1e6, 1), "sample": f"{n1} full calls"}
    # the other workloads, one whole call each on all threads
    per = {}
    for c in (1, 2, 3, 4):
        if c == cfg:
            continue
        dc = wl.make_config(c)
        tc = time.perf_counter()
        oracle.quant_act_fp4(dc["x"])
        oracle.gemm_lowrank(dc["x"], dc["wcode"], dc["wscales"], dc["g"], dc["V"], dc["U"],
                            dc["alpha"])
        tc = time.perf_counter() - tc
        bc = algorithmic_bytes(dc["M"], dc["N"], dc["K"], dc["r"])
        per[f"config{c}"] = {"us_per_call": round(tc * 1e6, 1), "GBps": round(bc / tc / 1e9, 4),
                             "cores": threads, "sample": "1 full call"}
    res["per_config"] = per
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=1, help="workload the step runs (default 1)")
    ap.add_argument("--rank", type=int, default=None,
                    help="run the workload at this rank instead of its own (0: the plain FP4 GEMM)")
    ap.add_argument("--schedule", type=int, default=0, help="BILOCO_SCHED_* (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the bench, run 10 device-to-device copies of BYTES bytes (the "
                         "known-size reference for HBM counters)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "this script into profiles/traffic_<schedule>_config<c>.json and .md")
    ap.add_argument("--busy-summary", metavar="PMC_DIR",
                    help="no GPU work: turn a rocprofv3 --pmc run of BUSY_COUNTERS into "
                         "profiles/busy_<schedule>_config<c>.json")
    ap.add_argument("--timeline", action="store_true",
                    help="per-wave stamps of one call of --config/--schedule, read from the "
                         "timeline build (libbiloco_tl.so); writes profiles/timeline_*.md")
    ap.add_argument("--timeline-r0", action="store_true", help="--timeline with r = 0")
    ap.add_argument("--timeline-step", action="store_true",
                    help="--timeline of the quantising call (biloco_gemm_lowrank_quant)")
    ap.add_argument("--only", choices=["weight-quant", "decompose", "stream-floor"],
                    help="time only this NEXT-row operation and print its JSON (for profiling)")
    args = ap.parse_args()
    if args.traffic_summary:
        return traffic_summary(args)
    if args.timeline:
        return timeline(args)
    if args.busy_summary:
        return busy_summary(args)
    if args.only:
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        res = (weight_quant_table() if args.only == "weight-quant" else
               decompose_time() if args.only == "decompose" else stream_floor())
        print(json.dumps({args.only: res}), flush=True)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(use --gpus 1).", file=sys.stderr)
        return 2

    import torch
    from bit_weight_gemm_amd import binding as B
    from bit_weight_gemm_amd import workloads as wl
    from bit_weight_gemm_amd.problem import DeviceProblem

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    src_hash = source_hash()
    cfg = args.config
    d = wl.make_config(cfg, r=args.rank)
    prob = DeviceProblem(d)
    M, N, K, r = prob.M, prob.N, prob.K, prob.r
    sched = args.schedule or B.biloco_default_schedule(M, N, K, r)
    sched_name = SCHED_NAMES.get(sched, str(sched))
    n_sets = max(2, int(ROT_BYTES // weight_bytes(prob)) + 1)
    rot = Rotation(prob, min(n_sets, args.steps))

    # warmup: W eager steps
    for i in range(args.warmup):
        prob.gemm_quant(sched, **rot.kw(i))
    torch.cuda.synchronize()

    # the timed region: exactly K steps, captured once, replayed once; a step
    # is biloco_gemm_lowrank_quant: the activation's FP4 quantisation and the
    # product (the quantisation rides in the z launch where there is one)
    K_steps = args.steps
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for i in range(K_steps):
            prob.gemm_quant(sched, stream=st, **rot.kw(i))
    graph.replay()                       # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu = e0.elapsed_time(e1) / 1e3
    ms_per_step = wall * 1e3 / K_steps
    nbytes = algorithmic_bytes(M, N, K, r)
    value = nbytes / (wall / K_steps) / 1e9

    # the product call alone (the dominant work), same rotation, events on its stream
    t_call = gemm_call_time(prob, sched, rot, min(K_steps, 400))
    achieved = nbytes / t_call / 1e9
    t_warm = gemm_call_time(prob, sched, None, 200)
    traffic = measured_traffic(cfg, sched_name) if args.rank is None else None

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded generators; weights rotated over >= 1.2 GB)",
        "config": {"workload": d["name"], "M": M, "K": K, "N": N, "r": r,
                   "schedule": sched_name, "global_batch": M, "parallelism": "none (1 GPU)"},
        "us_per_step": round(wall * 1e6 / K_steps, 3),
        "us_per_call": round(t_call * 1e6, 3),
        "us_per_call_cache_resident": round(t_warm * 1e6, 3),
        "pct_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "step_gpu_us": round(gpu * 1e6 / K_steps, 3),
        "roofline": {"bound": "hbm", "kernel": f"biloco_gemm_lowrank call ({sched_name}: "
                                               f"{CALL_KERNELS.get(sched_name, 'its launches')})",
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "bytes_per_call": nbytes},
        "source_hash": src_hash,
    }

    # the floors of this byte count: a launch that only reads it, an empty launch
    fl = stream_floor(configs=(cfg,), calls=200) if cfg in (1, 2, 3, 4) and args.rank is None else None
    if fl:
        out["stream_floor"] = {"read_us_per_call": fl[f"config{cfg}"]["us_per_call"],
                               "read_GBps": fl[f"config{cfg}"]["GBps"],
                               "empty_launch_us": fl["empty_launch_us"],
                               "call_over_read_floor": round(t_call * 1e6 / fl[f"config{cfg}"]["us_per_call"], 3)}

    if not args.no_configs:
        table = {}
        # correction overhead at this config: the same x and R with r = 0
        d0 = wl.make_config(cfg, r=0)
        p0 = DeviceProblem(d0)
        rot0 = Rotation(p0, max(2, int(ROT_BYTES // weight_bytes(p0)) + 1))
        s0 = B.biloco_default_schedule(M, N, K, 0)
        t0c = gemm_call_time(p0, s0, rot0, 400)
        out["r0_us_per_call"] = round(t0c * 1e6, 3)
        out["correction_overhead"] = round(t_call / t0c - 1.0, 4)
        del rot0, p0
        for c in (1, 2, 3, 4):
            dc = wl.make_config(c)
            pc = DeviceProblem(dc)
            sc = B.biloco_default_schedule(pc.M, pc.N, pc.K, pc.r)
            rc = Rotation(pc, max(2, int(ROT_BYTES // weight_bytes(pc)) + 1))
            calls = 100 if pc.M <= 2 else 20
            tc = gemm_call_time(pc, sc, rc, calls)
            # the same product as separate launches (plain product, z, correction)
            tcomp = gemm_call_time(pc, B.BILOCO_SCHED_COMPOSED, rc, calls)
            tcm = gemm_call_time(pc, B.BILOCO_SCHED_COMPOSED_MFMA, rc, calls)
            # the matrix-core schedules side by side (z in a launch of its own,
            # and every workgroup computing a tile of z at entry)
            mfma_times = {}
            for ms in (B.BILOCO_SCHED_FUSED_MFMA, B.BILOCO_SCHED_MFMA_ALLWG, B.BILOCO_SCHED_MFMA_SIDE,
                       B.BILOCO_SCHED_MFMA_ZEPI):
                if ms in B.biloco_schedules_for(pc.M, pc.N, pc.K, pc.r):
                    mfma_times[SCHED_NAMES[ms] + "_us_per_call"] = round(
                        gemm_call_time(pc, ms, rc, calls) * 1e6, 3)
            bc = algorithmic_bytes(pc.M, pc.N, pc.K, pc.r)
            del rc, pc
            torch.cuda.empty_cache()
            # the same x and R with r = 0, for the correction's cost at this shape
            pz = DeviceProblem(wl.make_config(c, r=0))
            rz = Rotation(pz, max(2, int(ROT_BYTES // weight_bytes(pz)) + 1))
            tz = gemm_call_time(pz, B.biloco_default_schedule(pz.M, pz.N, pz.K, 0), rz, calls)
            del rz, pz
            torch.cuda.empty_cache()
            flc = stream_floor(configs=(c,), calls=100)[f"config{c}"]
            table[f"config{c}"] = {"M": dc["M"], "K": dc["K"], "N": dc["N"], "r": dc["r"],
                                   "read_floor_us_per_call": flc["us_per_call"],
                                   "call_over_read_floor": round(tc * 1e6 / flc["us_per_call"], 3),
                                   "schedule": SCHED_NAMES.get(sc, sc),
                                   "us_per_call": round(tc * 1e6, 3),
                                   "GBps": round(bc / tc / 1e9, 1),
                                   "pct_peak": round(100 * bc / tc / 1e9 / PEAK_HBM_GBS, 2),
                                   "r0_us_per_call": round(tz * 1e6, 3),
                                   "correction_overhead": round(tc / tz - 1.0, 4),
                                   "composed_us_per_call": round(tcomp * 1e6, 3),
                                   "composed_mfma_us_per_call": round(tcm * 1e6, 3),
                                   "speedup_vs_composed": round(min(tcomp, tcm) / tc, 3),
                                   **mfma_times}
        out["per_config"] = table
        out["weight_quant"] = weight_quant_table()
        out["decompose"] = decompose_time()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
    return 0


def _pmc_rows(directory: str):
    """(kernel name, counter name, value) of every dispatch in a rocprofv3
    counter-collection CSV under `directory`."""
    import csv
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    rows = []
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                rows.append((row["Kernel_Name"], row["Counter_Name"], float(row["Counter_Value"])))
    return rows


TL_SLOTS = {
    "gemv": ["start", "first row's loads issued", "every row's loads issued", "rows done",
             "z values checked", "correction started", "stored"],
    "mfma": ["start", "loads issued", "z tile counted in", "activation decoded", "row block 0 done",
             "finisher known", "finisher done", "last row-block slot", "row blocks done",
             "first correction word ready", "correction done", "stored"],
}


def timeline(args) -> int:
    """Per-wave stamps (100 MHz real-time counter, in us from the earliest
    workgroup start) of the last call of a graph of 20 calls over rotated
    weights, from the timeline build of the library: quantiles over waves per
    named point, printed as JSON and written to profiles/timeline_<schedule>_
    <workload>.md with the command that made it."""
    import ctypes
    import numpy as np
    import torch
    from bit_weight_gemm_amd import binding as B
    from bit_weight_gemm_amd import build as hb
    from bit_weight_gemm_amd import workloads as wl
    from bit_weight_gemm_amd.problem import DeviceProblem
    if not os.path.exists(hb.TL_LIB):
        raise SystemExit(f"{hb.TL_LIB} is missing: build it with __graft_entry__.build()")
    B.LIB_PATH = hb.TL_LIB
    L = B.lib()
    cfg = args.config
    d = wl.make_config(cfg, r=0 if args.timeline_r0 else None)
    sched = args.schedule or B.biloco_default_schedule(d["M"], d["N"], d["K"], d["r"])
    step = args.timeline_step
    p = DeviceProblem(d, quantize=not step)
    rot = Rotation(p, 20)

    def one(i, st):
        if step:
            p.gemm_quant(sched, stream=st, **rot.kw(i))
        else:
            p.gemm(sched, stream=st, **rot.kw(i))
    t, g = time_graph(one, 20)
    fam = "gemv" if sched in (1, 2) and d["M"] <= 2 else "mfma"
    zero = getattr(L, f"biloco_tl_{fam}_zero")
    read = getattr(L, f"biloco_tl_{fam}_read")
    read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    torch.cuda.synchronize()
    assert zero() == 0
    g.replay()
    torch.cuda.synchronize()
    n = 4096 * 8 * 16
    buf = np.zeros(n, np.uint64)
    assert read(buf.ctypes.data, n) == 0
    tl = buf.reshape(4096, 8, 16).astype(np.int64)
    wgs = np.nonzero(tl[:, 0, 0])[0]
    tl = tl[wgs]
    t0 = tl[:, :, 0][tl[:, :, 0] > 0].min()
    rel = np.where(tl > 0, (tl - t0) * 0.01, np.nan)
    names = TL_SLOTS[fam]
    groups = {}
    if fam == "gemv":
        stream_wg = tl[:, 0, 1] > 0
        groups["stream workgroups"] = (stream_wg, range(len(names)))
        if (~stream_wg).any():
            groups["side workgroups"] = (~stream_wg, [0, 2])
    else:
        ze = tl[:, 0, 14] == 1          # the z-in-epilogue schedule's side workgroups
        prod = (tl[:, 0, 1] > 0) & ~ze  # side workgroups stream no rows
        groups["product workgroups"] = (prod, [k for k in range(len(names)) if k != 6])
        if (~prod & ~ze).any():
            groups["side workgroups"] = (~prod & ~ze, [0, 3, 4, 5, 6, 2])
        if ze.any():
            groups["z-in-epilogue side workgroups"] = (ze, [0, 1, 2, 3, 4, 5])
        fin = tl[:, 0, 12] == 1
        if fin.any():
            groups["finisher workgroups"] = (fin, [6])
    out = {"config": cfg, "r": d["r"], "schedule": SCHED_NAMES.get(sched, sched),
           "call": "quantise + product" if step else "product", "us_per_call_timeline_build":
           round(t * 1e6, 3), "workgroups": int(len(wgs)), "groups": {}}
    if fam == "gemv" and (tl[:, :, 8] > 0).any():
        # one launch: the stream waves' z values by the read that had the tag
        cnt = {k: int((tl[:, :, s] - 1)[tl[:, :, s] > 0].sum()) for k, s in
               (("first read", 8), ("second read", 9), ("read again", 10))}
        out["z_reads"] = cnt
    if fam == "mfma":
        out["finishers"] = int((tl[:, 0, 12] == 1).sum())
        out["waves_computing_z_locally"] = int((tl[:, :, 13] == 1).sum())
    for gname, (mask, slots) in groups.items():
        rows = {}
        for k in slots:
            v = rel[mask, :, k].ravel()
            v = v[~np.isnan(v)]
            label = names[k]
            if gname.startswith("z-in-epilogue"):
                label = {0: "start", 1: "x and V part staged in LDS", 2: "part's MFMAs done",
                         3: "partials stored", 4: "every part counted in", 5: "words finished"}[k]
            elif gname.startswith("side"):
                label = {2: "z published" if fam == "gemv" else "z words published",
                         3: "first word: first loads issued", 4: "first word: first loads used",
                         5: "first word: second loads used", 6: "first word: waves' sums in LDS"}.get(k, label)
            if v.size:
                rows[label] = {q: round(float(np.percentile(v, pc)), 2) for q, pc in
                                  (("min", 0), ("p10", 10), ("median", 50), ("p90", 90), ("max", 100))}
                rows[label]["waves"] = int(v.size)
        out["groups"][gname] = rows
    if fam == "mfma" and prod.any():
        # where the product's time goes: by wave index inside the workgroup,
        # the spread between a workgroup's first and last wave, and by XCD
        # (workgroup b runs on XCD b % 8)
        kd, ks = names.index("row blocks done"), names.index("stored")
        done = rel[prod, :, kd]
        spread = np.nanmax(done, axis=1) - np.nanmin(done, axis=1)
        xcd = wgs[prod] % 8
        out["product_breakdown"] = {
            "row_blocks_done_median_by_wave": [round(float(np.nanmedian(done[:, w])), 2) for w in range(8)],
            "within_workgroup_spread_us": {q: round(float(np.nanpercentile(spread, pc)), 2) for q, pc in
                                           (("p10", 10), ("median", 50), ("p90", 90))},
            "stored_median_by_xcd": [round(float(np.nanmedian(rel[prod, 0, ks][xcd == x])), 2)
                                     if (xcd == x).any() else None for x in range(8)]}
    if fam == "gemv":
        # the stream waves' rows by wave index inside the workgroup (wave w
        # is the (w // 4 + 1)-th wave of SIMD w % 4) and the spread inside a
        # workgroup
        sw = tl[:, 0, 1] > 0
        done = rel[sw, :, names.index("rows done")]
        if np.isfinite(done).any():
            spread = np.nanmax(done, axis=1) - np.nanmin(done, axis=1)
            out["stream_breakdown"] = {
                "rows_done_median_by_wave": [round(float(np.nanmedian(done[:, w])), 2) for w in range(8)],
                "within_workgroup_spread_us": {q: round(float(np.nanpercentile(spread, pc)), 2) for q, pc in
                                               (("p10", 10), ("median", 50), ("p90", 90))}}
    cmd = "python3 bench.py --timeline --config %d%s%s%s" % (
        cfg, f" --schedule {args.schedule}" if args.schedule else "",
        " --timeline-r0" if args.timeline_r0 else "", " --timeline-step" if step else "")
    wname = f"M{d['M']}_K{d['K']}_N{d['N']}_r{d['r']}"
    lines = [f"# Timeline: {out['schedule']}, {out['call']}, M={d['M']} K={d['K']} N={d['N']} r={d['r']}", "",
             "Command (repository root, one MI355X, after `__graft_entry__.build()`):", "", "```", cmd, "```", "",
             "Per-wave stamps of the 100 MHz real-time counter at named points of the kernel "
             "(the library built with BILOCO_TIMELINE), for the last call of a graph of 20 calls over "
             "rotated weights; microseconds from the earliest workgroup start.  The stamps' stores "
             f"slow the call a little: {out['us_per_call_timeline_build']} us per call in this build.", ""]
    if "z_reads" in out:
        zr = out["z_reads"]
        lines += ["z values of the stream waves by the read that carried the call's tag: "
                  + "; ".join(f"{k} {v}" for k, v in zr.items()) + ".", ""]
    if fam == "mfma":
        lines += [f"Finisher workgroups: {out['finishers']}; waves that computed z locally: "
                  f"{out['waves_computing_z_locally']}.", ""]
    for gname, rows in out["groups"].items():
        lines += [f"## {gname}", "", "| point | waves | min | p10 | median | p90 | max |",
                  "|---|---:|---:|---:|---:|---:|---:|"]
        for k, v in rows.items():
            lines.append(f"| {k} | {v['waves']} | {v['min']} | {v['p10']} | {v['median']} | {v['p90']} | {v['max']} |")
        lines.append("")
    if "product_breakdown" in out:
        pb = out["product_breakdown"]
        lines += ["## product workgroups: where the time goes", "",
                  "- row blocks done, median by wave index 0..7: " +
                  ", ".join(str(v) for v in pb["row_blocks_done_median_by_wave"]),
                  "- spread between a workgroup's first and last wave to finish its row blocks (p10 / median / p90): "
                  + " / ".join(str(v) for v in pb["within_workgroup_spread_us"].values()),
                  "- stored, median by XCD 0..7: " + ", ".join(str(v) for v in pb["stored_median_by_xcd"]), ""]
    if "stream_breakdown" in out:
        sb = out["stream_breakdown"]
        lines += ["## stream workgroups: where the time goes", "",
                  "- rows done, median by wave index 0..7: " +
                  ", ".join(str(v) for v in sb["rows_done_median_by_wave"]),
                  "- spread between a workgroup's first and last wave to finish its rows (p10 / median / p90): "
                  + " / ".join(str(v) for v in sb["within_workgroup_spread_us"].values()), ""]
    tag = "_step" if step else ""
    path = os.path.join(ROOT, "profiles", f"timeline_{out['schedule']}_{wname}{tag}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(out), flush=True)
    return 0


BUSY_COUNTERS = ["GRBM_GUI_ACTIVE", "GRBM_COUNT", "SQ_BUSY_CU_CYCLES", "SQ_ACTIVE_INST_VALU",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_CYCLES"]


def busy_summary(args) -> int:
    """Busy counters per product launch from one rocprofv3 --pmc run of this
    script (BUSY_COUNTERS, one pass): per kernel, the median over its
    dispatches of each counter, and three ratios.

    Units as the counters read on MI355X (8 XCDs, 32 CUs and 4 shader engines
    each): GRBM_GUI_ACTIVE is summed over the XCDs and SQ_CYCLES over the
    shader engines (it reads 4 GRBM_GUI_ACTIVE for every kernel);
    SQ_BUSY_CU_CYCLES is clock cycles summed over the 256 CUs;
    SQ_VALU_MFMA_BUSY_CYCLES is cycles summed over the 1024 SIMDs (a
    16x16x32 f16 MFMA adds 16); SQ_ACTIVE_INST_VALU is quad-cycles summed
    over the SIMDs.
      cu_busy_us  = SQ_BUSY_CU_CYCLES / 256 / 2400 MHz: the time an average
                    CU had work of the kernel (the profiler's GUI window,
                    window_us, also holds the dispatch set-up);
      mfma_frac   = SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES): the
                    matrix cores' share of the SIMD cycles while CUs were busy;
      valu_frac   = 4 SQ_ACTIVE_INST_VALU / (4 SQ_BUSY_CU_CYCLES): the same
                    for vector ALU instructions."""
    import statistics
    from bit_weight_gemm_amd import workloads as wl
    from bit_weight_gemm_amd import binding as B
    directory = args.busy_summary
    cfg = args.config
    d = wl.make_config(cfg)
    sched = args.schedule or B.biloco_default_schedule(d["M"], d["N"], d["K"], d["r"])
    sched_name = SCHED_NAMES.get(sched, str(sched))
    per = {}
    for k, c, v in _pmc_rows(directory):
        if "biloco::" in k and "quant_act" not in k and "pack_signs" not in k:
            per.setdefault(k.split("(")[0], {}).setdefault(c, []).append(v)
    kernels = {}
    for k, cs in per.items():
        med = {c: statistics.median(v) for c, v in cs.items()}
        row = {"counters": med}
        if med.get("GRBM_GUI_ACTIVE"):
            row["window_us"] = round(med["GRBM_GUI_ACTIVE"] / 8 / 2400, 3)
        busy = med.get("SQ_BUSY_CU_CYCLES")
        if busy:
            row["cu_busy_us"] = round(busy / 256 / 2400, 3)
            row["mfma_frac"] = round(med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (4 * busy), 4)
            row["valu_frac"] = round(med.get("SQ_ACTIVE_INST_VALU", 0) / busy, 4)
        kernels[k] = row
    out = {"config": cfg, "schedule": sched_name, "source_hash": source_hash(sched_name),
           "counters": BUSY_COUNTERS, "kernels": kernels}
    with open(os.path.join(ROOT, "profiles", f"busy_{sched_name}_config{cfg}.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


def _is_step_variant(name: str) -> bool:
    """fused_gemv_kernel<MM, KBL, ZMODE, true>: the launch that quantises the
    activation itself (a step), not the product call's kernel."""
    return "fused_gemv_kernel<" in name and name.rstrip().endswith("true>")


def traffic_summary(args) -> int:
    """HBM bytes per product call from rocprofv3 --pmc runs of this script.

    FETCH_SIZE and WRITE_SIZE are per-dispatch counters in KiB.  They are
    scaled by the same counter over the known-size copy run at the end
    (--copy-calibration): factor = copy bytes / (counter of the copy kernel).
    The product call's traffic is the sum over its kernels (every dispatch
    name that holds biloco:: but not the activation quantiser or the packer)."""
    import statistics
    from bit_weight_gemm_amd import workloads as wl
    fetch_dir, write_dir = args.traffic_summary
    cfg = args.config
    d = wl.make_config(cfg)
    copy_bytes = args.copy_calibration
    if not copy_bytes:
        raise SystemExit("--traffic-summary needs the --copy-calibration size the runs used")
    res = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _pmc_rows(directory) if r[1] == counter]
        copies = [v for k, c, v in rows if "copy" in k.lower() or "elementwise" in k.lower()]
        big = sorted(copies)[-10:] if copies else []
        if not big:
            raise SystemExit(f"no copy dispatch found for {counter}")
        kib_copy = statistics.median(big)
        factor = copy_bytes / kib_copy
        per_kernel = {}
        for k, c, v in rows:
            if "biloco::" in k and "quant_act" not in k and "pack_signs" not in k:
                per_kernel.setdefault(k.split("(")[0], []).append(v)
        kernels = {k: statistics.median(v) * factor for k, v in per_kernel.items()}
        # the one-launch M <= 2 kernel has a variant that also quantises the
        # activation (the step's); the call launches the other one
        call = {k: b for k, b in kernels.items() if not _is_step_variant(k)}
        res[counter] = {"factor_bytes_per_unit": factor, "copy_units_median": kib_copy,
                        "per_kernel_bytes": kernels, "call_bytes": sum(call.values())}
    bytes_per_call = res["FETCH_SIZE"]["call_bytes"] + res["WRITE_SIZE"]["call_bytes"]
    sched_name = args.sched_name if hasattr(args, "sched_name") else None
    from bit_weight_gemm_amd import binding as B
    sched = args.schedule or B.biloco_default_schedule(d["M"], d["N"], d["K"], d["r"])
    sched_name = SCHED_NAMES.get(sched, str(sched))
    nb = algorithmic_bytes(d["M"], d["N"], d["K"], d["r"])
    out = {"config": cfg, "schedule": sched_name, "source_hash": source_hash(sched_name),
           "bytes_per_call": round(bytes_per_call), "algorithmic_bytes": nb,
           "ratio_to_algorithmic": round(bytes_per_call / nb, 4),
           "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
           "copy_calibration_bytes": copy_bytes}
    base = os.path.join(ROOT, "profiles", f"traffic_{sched_name}_config{cfg}")
    with open(base + ".json", "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
