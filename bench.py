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
               5: "composed_mfma"}
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
                              "mfma_product_kernel + mfma_epilogue_kernel (split K)"}


def source_hash() -> str:
    """Hash of the kernel and library sources' code (comments excluded)."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bit_weight_gemm_amd", "csrc", "*"))):
        with open(f, "r", encoding="utf-8") as fh:
            h.update(os.path.basename(f).encode())
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg: int, sched_name: str, src_hash: str):
    """HBM bytes per call from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{sched_name}_config{cfg}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash:
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
    """biloco_peel_decompose on a seeded fp32 weight of the config-1 shape: one
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
            "bytes": nbytes}


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
    return {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "us_per_call": round(dt * 1e6, 1),
            "sample": f"{n} full calls of the config-{cfg} product on the host (quantise x, then "
                      f"y in fp64 over all M*N outputs), same seeded inputs as the GPU"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=1, help="workload the step runs (default 1)")
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
    ap.add_argument("--only", choices=["weight-quant", "decompose"],
                    help="time only this NEXT-row operation and print its JSON (for profiling)")
    args = ap.parse_args()
    if args.traffic_summary:
        return traffic_summary(args)
    if args.only:
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        res = weight_quant_table() if args.only == "weight-quant" else decompose_time()
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
    d = wl.make_config(cfg)
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
    traffic = measured_traffic(cfg, sched_name, src_hash)

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
            bc = algorithmic_bytes(pc.M, pc.N, pc.K, pc.r)
            del rc, pc
            torch.cuda.empty_cache()
            # the same x and R with r = 0, for the correction's cost at this shape
            pz = DeviceProblem(wl.make_config(c, r=0))
            rz = Rotation(pz, max(2, int(ROT_BYTES // weight_bytes(pz)) + 1))
            tz = gemm_call_time(pz, B.biloco_default_schedule(pz.M, pz.N, pz.K, 0), rz, calls)
            del rz, pz
            torch.cuda.empty_cache()
            table[f"config{c}"] = {"M": dc["M"], "K": dc["K"], "N": dc["N"], "r": dc["r"],
                                   "schedule": SCHED_NAMES.get(sc, sc),
                                   "us_per_call": round(tc * 1e6, 3),
                                   "GBps": round(bc / tc / 1e9, 1),
                                   "pct_peak": round(100 * bc / tc / 1e9 / PEAK_HBM_GBS, 2),
                                   "r0_us_per_call": round(tz * 1e6, 3),
                                   "correction_overhead": round(tc / tz - 1.0, 4),
                                   "composed_us_per_call": round(tcomp * 1e6, 3),
                                   "composed_mfma_us_per_call": round(tcm * 1e6, 3),
                                   "speedup_vs_composed": round(min(tcomp, tcm) / tc, 3)}
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
        res[counter] = {"factor_bytes_per_unit": factor, "copy_units_median": kib_copy,
                        "per_kernel_bytes": kernels, "call_bytes": sum(kernels.values())}
    bytes_per_call = res["FETCH_SIZE"]["call_bytes"] + res["WRITE_SIZE"]["call_bytes"]
    sched_name = args.sched_name if hasattr(args, "sched_name") else None
    from bit_weight_gemm_amd import binding as B
    sched = args.schedule or B.biloco_default_schedule(d["M"], d["N"], d["K"], d["r"])
    sched_name = SCHED_NAMES.get(sched, str(sched))
    nb = algorithmic_bytes(d["M"], d["N"], d["K"], d["r"])
    out = {"config": cfg, "schedule": sched_name, "source_hash": source_hash(),
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
