#!/usr/bin/env python3
"""Benchmark of the MoE Q4_0 x Q8_1 expert matmul on one MI355X.

One step = the whole hot path over one batch: Q8_1 quantisation of the fp32
activations, routing (bucketing of the (token, top-k) pairs by expert) and the
expert matmul, through the C ABI of libftq.  Workload: the FreeToken PR #185
"Performance" shape (128 experts, nrows N = 1408, hidden K = 2816, top_k = 8)
at T = 8191 tokens (65528 pairs), seeded synthetic inputs (weights N(0, 0.02),
activations N(0, 1), uniform distinct routing).  Inputs are resident in HBM
before timing starts.

    python bench.py [--steps K] [--warmup W] [--T tokens]
    python bench.py --workload page1_down  # the second layer: per-pair rows + combine
    python bench.py --workload page1_act   # the first layer with act(gate) * up fused
    python bench.py --workload mixtral --T 1 --wtype q8_0   # another GGUF weight type (random valid blocks)
    python bench.py --mode profile         # a short run for rocprofv3
    python bench.py --summarize-pmc DIR    # HBM traffic from rocprofv3 --pmc runs
    python bench.py --summarize-trace DB   # kernel table from a rocprofv3 --kernel-trace database

Prints one JSON line.  `value` is milliseconds per step (lower is better),
wall clock over the timed steps with the inputs resident in HBM (warm caches);
`step_ms` gives the median, minimum and maximum of the same steps from HIP
events, warm and cold (each cold step after a 1 GiB write that evicts the L2
and the 256 MB last-level cache); `roofline` reports the dominant kernel (the
grouped matmul: against the dense int8 MFMA peak, its block products run on
int8 MFMAs) using its algorithmic operation count, timed with HIP events on the
stream it runs on; `decode` adds the GEMV path at Mixtral-8x7B decode shapes
(T = 1 and 8) against the HBM roofline, warm and cold; `sweep` times one
routed matmul call of the page-1 shape at T = 1 .. 8192 on the path that
FTQ_PATH_AUTO takes, against both rooflines; `cpu_baseline` is the CPU oracle
on a bounded sample of the same workload, with the host CPU named.
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE Q4_0xQ8_1 matmul time (ms) + HBM GB/s / int8 MFMA % at T=1..8192, top_k=8"
WORKLOAD = dict(workload="freetoken_pr185_moe_q4_0", E=128, N=1408, K=2816, top_k=8, routing="uniform", seed=0)
DEFAULT_T = 8191
# Other shapes the paths are checked on, for profiling a path at its real shape
# (`--workload`); the bench line proper is the page-1 workload above.
# A "down" workload is the second layer of the expert FFN: one Q8_1 row per
# (token, slot) pair in, the expert width as K and the hidden size as N, then
# the per-token router-weighted combine of the k pair outputs.  An "act"
# workload is the first layer with its gated activation fused: N weight rows
# per expert (gate rows, then up rows), output act(gate) * up of width N/2.
WORKLOADS = {
    "page1": (WORKLOAD, DEFAULT_T),
    "mixtral": (dict(workload="mixtral_8x7b_up", E=8, N=14336, K=4096, top_k=2, routing="uniform", seed=0), 8),
    "qwen": (dict(workload="qwen3_30b_a3b_up", E=128, N=768, K=2048, top_k=8, routing="zipf", seed=0), 8192),
    "page1_down": (dict(workload="freetoken_pr185_moe_q4_0_down", layer="down", E=128, N=2816, K=1408, top_k=8,
                        routing="uniform", seed=0), DEFAULT_T),
    "mixtral_down": (dict(workload="mixtral_8x7b_down", layer="down", E=8, N=4096, K=14336, top_k=2,
                          routing="uniform", seed=0), 8),
    "qwen_down": (dict(workload="qwen3_30b_a3b_down", layer="down", E=128, N=2048, K=768, top_k=8,
                       routing="zipf", seed=0), 8192),
    "page1_act": (dict(workload="freetoken_pr185_moe_q4_0_gelu_tanh_and_mul", layer="act", act="gelu_tanh", E=128,
                       N=1408, K=2816, top_k=8, routing="uniform", seed=0), DEFAULT_T),
    "mixtral_act": (dict(workload="mixtral_8x7b_gate_up_silu", layer="act", act="silu", E=8, N=28672, K=4096,
                         top_k=2, routing="uniform", seed=0), 8),
    "qwen_act": (dict(workload="qwen3_30b_a3b_gate_up_silu", layer="act", act="silu", E=128, N=1536, K=2048,
                      top_k=8, routing="zipf", seed=0), 8192),
}
# The pages' own measurement of this workload: the fixed GEMV kernel at 8191
# tokens on a Tesla T4 (FreeToken PR #185, Performance), the faster of two runs.
PAGES_MS_T8191 = 705.8
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
F16_PEAK_TFLOPS = 2500.0        # MI355X dense fp16 MFMA (context: the fp16 formulation's ceiling)
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA (the grouped kernel's block products)
DOMINANT = "moe_grouped_kernel"
SCRUB_BYTES = 1 << 30           # written before each cold step: larger than the L2s and the 256 MB MALL
# decode records carried on every bench line: the GEMV at Mixtral-8x7B's
# up-projection shape (mlxcel PR #652, Summary) at one and eight tokens
DECODE = (("mixtral", 1), ("mixtral", 8))
# the metric's batch range on the page-1 shape (one routed matmul call per
# point, FTQ_PATH_AUTO): decode, mid-range and prefill sizes
SWEEP_T = (1, 8, 32, 128, 512, 2048, 8192)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _stats(xs):
    return {"median": round(statistics.median(xs), 4), "min": round(min(xs), 4), "max": round(max(xs), 4),
            "n": len(xs)}


def _cold_times(fn, scrub, reps):
    """HIP-event time of fn() right after a write of the scrub buffer, reps
    times.  The scrub keeps the GPU busy while the host enqueues fn, so the
    events bracket fn's kernels, not host submission."""
    import torch
    out = []
    for i in range(reps):
        scrub.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def decode_record(name: str, T: int, scrub, reps: int = 10) -> dict:
    """The GEMV path at a decode shape: one routed matmul call, warm (graph of
    20 calls, per call, 5 replays) and cold (after a 1 GiB scrub, reps calls),
    against the HBM roofline of its algorithmic bytes."""
    import numpy as np
    import torch
    from quantized_moe_expert_quantize_amd import ftq, inputs
    wl, _ = WORKLOADS[name]
    E, N, K, k = wl["E"], wl["N"], wl["K"], wl["top_k"]
    dev = scrub.device
    # weights N(0, 0.02) from torch's seeded device generator, Q4_0 by libftq
    # (the GEMV's time does not depend on the values; this keeps set-up short)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl["seed"])
    wq = torch.empty((E, N, K // 32 * 18), dtype=torch.uint8, device=dev)
    for e in range(E):
        w = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
        wq[e] = ftq.quantize_q4_0(w).view(N, K // 32 * 18)
        del w
    ids = inputs.routing(T, E, k, seed=wl["seed"], kind=wl["routing"])
    aq = ftq.quantize_q8_1(torch.from_numpy(inputs.activations(T, K, seed=wl["seed"])).to(dev))
    ids_d = torch.from_numpy(ids).to(dev)
    path = ftq.select_path(E, N, K, T, k)
    out = torch.empty((T * k, N), dtype=torch.float32, device=dev)
    need = ftq.workspace_bytes(E, N, K, T, k, path)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev) if need else None
    ftq.moe_route(ids_d, E, ws, path)

    def call():
        ftq.moe_routed(wq, aq, ids_d, E, N, K, out, ws, path)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    R = 20
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(R):
            call()
    torch.cuda.synchronize()
    warm = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        warm.append(a.elapsed_time(b) / R)
    cold = _cold_times(call, scrub, reps)
    alg = _algorithmic_bytes(E, N, K, T, k, ids)
    wm, cm = statistics.median(warm), statistics.median(cold)
    traffic = None
    tf = traffic_file("moe_gemv_kernel" if path == ftq.PATH_GEMV else "moe_grouped_kernel", name, T)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("lib_sha256") == _lib_hash() and rec.get("T") == T:
            traffic = rec.get("bytes_per_launch")
    return {"workload": wl["workload"], "T": T, "pairs": T * k, "path": {1: "gemv", 2: "grouped"}[path],
            "kernel": "moe_gemv_kernel" if path == ftq.PATH_GEMV else "moe_grouped_kernel",
            "alg_bytes_per_launch": alg,
            "warm_us": {k_: round(v * 1e3, 2) for k_, v in _stats(warm).items() if k_ != "n"},
            "cold_us": {k_: round(v * 1e3, 2) for k_, v in _stats(cold).items() if k_ != "n"},
            "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "achieved_warm": round(alg / (wm / 1e3) / 1e9, 1),
                         "frac_warm": round(alg / (wm / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                         "achieved_cold": round(alg / (cm / 1e3) / 1e9, 1),
                         "frac_cold": round(alg / (cm / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": traffic},
            "timing": "warm: HIP events around a graph replay of 20 calls, per call, 5 replays; cold: HIP events "
                      f"around one call right after a 1 GiB write, {reps} calls"}


def sweep_record(scrub) -> dict:
    """The page-1 shape (128 experts, N = 1408, K = 2816, top_k = 8) over the
    metric's batch range: per T one routed matmul call on the path that
    FTQ_PATH_AUTO takes, warm (HIP events around a graph of R calls, per call,
    median of 5 replays), with its algorithmic bytes and operations against the
    HBM and the int8 MFMA roofline (the path's own bound first)."""
    import torch
    from quantized_moe_expert_quantize_amd import ftq, inputs
    wl, _ = WORKLOADS["page1"]
    E, N, K, k = wl["E"], wl["N"], wl["K"], wl["top_k"]
    dev = scrub.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl["seed"])
    wq = torch.empty((E, N, K // 32 * 18), dtype=torch.uint8, device=dev)
    for e in range(E):
        w = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
        wq[e] = ftq.quantize_q4_0(w).view(N, K // 32 * 18)
        del w
    points = []
    for T in SWEEP_T:
        ids = inputs.routing(T, E, k, seed=wl["seed"], kind=wl["routing"])
        aq = ftq.quantize_q8_1(torch.from_numpy(inputs.activations(T, K, seed=wl["seed"])).to(dev))
        ids_d = torch.from_numpy(ids).to(dev)
        path = ftq.select_path(E, N, K, T, k)
        out = torch.empty((T * k, N), dtype=torch.float32, device=dev)
        need = ftq.workspace_bytes(E, N, K, T, k, path)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev) if need else None
        ftq.moe_route(ids_d, E, ws, path)

        def call():
            ftq.moe_routed(wq, aq, ids_d, E, N, K, out, ws, path)

        for _ in range(3):
            call()
        torch.cuda.synchronize()
        R = 20 if T <= 512 else 4
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(R):
                call()
        torch.cuda.synchronize()
        per_call = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            per_call.append(a.elapsed_time(b) / R)
        ms = statistics.median(per_call)
        alg = _algorithmic_bytes(E, N, K, T, k, ids)
        ops = 2 * T * k * N * K
        gbs, tops = alg / (ms / 1e3) / 1e9, ops / (ms / 1e3) / 1e12
        gemv = path == ftq.PATH_GEMV
        points.append({"T": T, "pairs": T * k, "path": "gemv" if gemv else "grouped", "us": round(ms * 1e3, 2),
                       "alg_bytes": alg, "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                       "TOPS": round(tops, 2), "int8_frac": round(tops / INT8_PEAK_TOPS, 4),
                       "bound": "hbm" if gemv else "mfma"})
        del g, out, ws, aq, ids_d
    return {"workload": wl["workload"], "E": E, "N": N, "K": K, "top_k": k, "routing": wl["routing"],
            "timing": "one routed matmul call (FTQ_PATH_AUTO; routing excluded) per point: HIP events around a graph "
                      "replay of R calls (R = 20 up to T = 512, else 4), per call, median of 5 replays; inputs "
                      "resident (warm)",
            "points": points}


def traffic_file(kernel: str, workload: str, T: int) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_T{T}_traffic.json")


def _lib_hash() -> str:
    p = os.path.join(ROOT, "quantized_moe_expert_quantize_amd", "libftq.sha256")
    return open(p).read().strip() if os.path.exists(p) else ""


WTYPES = {"q4_0": 2, "q4_1": 3, "q5_0": 6, "q5_1": 7, "q8_0": 8}
W_BLOCK_BYTES = {2: 18, 3: 20, 6: 22, 7: 24, 8: 34}


def _algorithmic_bytes(E, N, K, T, k, ids, act_rows=None, out_cols=None, block_bytes=18):
    """Bytes the method must move: the distinct experts' Q4_0 rows, the Q8_1
    activations (one row per token, or per pair), the int32 ids and the fp32
    output (N columns, or N/2 with the activation fused)."""
    import numpy as np
    nb = K // 32
    rows = T if act_rows is None else act_rows
    cols = N if out_cols is None else out_cols
    distinct = len(np.unique(ids[(ids >= 0) & (ids < E)]))
    return distinct * N * nb * block_bytes + rows * nb * 36 + 4 * T * k + 4 * T * k * cols


def summarize_pmc(d: str, kernel: str = DOMINANT) -> None:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    into HBM bytes per launch of the dominant kernel, scaled by what the same
    counters read for a plain copy of known size (bench.py --mode profile runs
    one: 1 GiB read, 1 GiB written)."""
    import csv
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row.get("Kernel_Name", "")
                ctr = row.get("Counter_Name", "")
                v = float(row.get("Counter_Value", "nan"))
                # the calibration kernel is torch's x * 1.0 over 1 GiB (bench.py --mode profile)
                kind = "dominant" if kernel in name else ("copy" if "AUnaryFunctor" in name else None)
                if kind is None:
                    continue
                vals.setdefault((kind, ctr), []).append(v)
    out = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        dom = vals.get(("dominant", ctr))
        cp = vals.get(("copy", ctr))
        if not dom or not cp:
            continue
        copy_kib = statistics.median(cp)
        factor = (1 << 30) / (copy_kib * 1024.0)
        out[ctr] = dict(kib_per_dispatch=statistics.median(dom), copy_kib=copy_kib, factor=factor,
                        bytes_per_launch=statistics.median(dom) * 1024.0 * factor)
    fetch, write = out.get("FETCH_SIZE"), out.get("WRITE_SIZE")
    if fetch and write:
        out["bytes_per_launch"] = fetch["bytes_per_launch"] + write["bytes_per_launch"]
    print(json.dumps(out, indent=1))


def summarize_counters(d: str, kernel: str = DOMINANT) -> None:
    """Median per-dispatch value of every counter that rocprofv3 --pmc runs
    under d collected for the kernels whose name contains `kernel`, with the
    derived utilisations (SQ cycle counters are per SE summed; GRBM_GUI_ACTIVE
    is the kernel's GPU cycles)."""
    import csv
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if kernel not in row.get("Kernel_Name", ""):
                    continue
                key = (f, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                c = per.setdefault(row["Counter_Name"], {})
                c[key] = c.get(key, 0.0) + float(row["Counter_Value"])
    med = {c: statistics.median(v.values()) for c, v in per.items()}
    print("| counter | median per dispatch | dispatches |")
    print("|---|---|---|")
    for c in sorted(med):
        print(f"| {c} | {med[c]:.6g} | {len(per[c])} |")
    return med


def summarize_trace(db: str) -> None:
    """Per-kernel table (calls, total / average duration, registers, LDS, grid)
    from a rocprofv3 --kernel-trace database (rocpd SQLite)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, count(*), sum(duration), avg(duration), max(vgpr_count), max(accum_vgpr_count), "
        "max(sgpr_count), max(lds_size), max(grid_x), max(workgroup_x) from kernels group by name "
        "order by sum(duration) desc").fetchall()
    grand = sum(r[2] for r in rows) or 1
    print("| kernel | calls | total (us) | average (us) | % of GPU time | arch VGPR | AGPR | SGPR | LDS (B) "
          "| grid (work-items) | block |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for name, n, tot, avg, vg, ag, sg, lds, gx, wx in rows:
        short = name.replace("ftq::(anonymous namespace)::", "")
        short = short[5:] if short.startswith("void ") else short
        short = short.split("(")[0]
        print(f"| `{short}` | {n} | {tot / 1e3:.1f} | {avg / 1e3:.2f} | {100.0 * tot / grand:.1f} | {vg} | {ag} | {sg} "
              f"| {lds} | {gx} | {wx} |")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="page1")
    ap.add_argument("--T", type=int, default=None, help="tokens (default: the workload's own)")
    ap.add_argument("--mode", choices=["bench", "profile"], default="bench")
    ap.add_argument("--wtype", choices=sorted(WTYPES), default="q4_0",
                    help="weight block type (not q4_0: random valid blocks, plain layers only; q5_* on the GEMV path)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the Mixtral decode records")
    ap.add_argument("--no-sweep", action="store_true", help="skip the page-1 batch sweep (T = 1 .. 8192)")
    ap.add_argument("--cold-steps", type=int, default=10, help="steps timed after a 1 GiB cache scrub each")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192, help="tokens the CPU oracle runs (10-30 s on the box)")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--pmc-kernel", default=DOMINANT, help="kernel whose counters --summarize-pmc reports")
    ap.add_argument("--summarize-trace", metavar="DB", help="per-kernel table from a rocprofv3 --kernel-trace database")
    ap.add_argument("--summarize-counters", metavar="DIR", help="median per-dispatch counters of --pmc-kernel under DIR")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.pmc_kernel)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.pmc_kernel)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only; --gpus N with N > 1 is not supported "
              "(the pairs shard by expert or by weight rows across GPUs, but no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_moe_expert_quantize_amd import ftq, inputs

    wl, wl_T = WORKLOADS[args.workload]
    E, N, K, k = wl["E"], wl["N"], wl["K"], wl["top_k"]
    T = args.T if args.T is not None else wl_T
    seed = wl["seed"]
    down = wl.get("layer") == "down"
    fused = wl.get("layer") == "act"
    wt = WTYPES[args.wtype]
    if wt != 2 and fused:
        print("bench.py: the fused activation takes Q4_0 weights only", file=sys.stderr)
        sys.exit(2)
    act_kind = {"silu": 1, "gelu_tanh": 2}.get(wl.get("act", ""), 0)
    act_rows = T * k if down else T
    out_cols = N // 2 if fused else N
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    # ---- inputs, resident in HBM --------------------------------------------
    w32 = inputs.weights(E, N, K, seed=seed) if wt == 2 else None
    x32 = inputs.activations(act_rows, K, seed=seed)
    ids = inputs.routing(T, E, k, seed=seed, kind=wl["routing"])
    gates = inputs.gates(T, k, seed=seed)
    if wt == 2:
        wdev = torch.from_numpy(w32).to(dev)
        wq = ftq.quantize_q4_0(wdev)
        del wdev
    else:
        wq = torch.from_numpy(inputs.gguf_blocks(wt, E, N, K, seed=seed)).to(dev)
    x = torch.from_numpy(x32).to(dev)
    ids_d = torch.from_numpy(ids).to(dev)
    path = ftq.PATH_GEMV if wt in ftq.GEMV_ONLY else ftq.select_path(E, N, K, T, k)
    gates_d = torch.from_numpy(gates).to(dev)
    aq = torch.empty((act_rows, K // 32 * 36), dtype=torch.uint8, device=dev)
    out = torch.empty((T * k, out_cols), dtype=torch.float32, device=dev)
    comb = torch.empty((T, N), dtype=torch.float32, device=dev) if down else None
    need = (ftq.pairs_workspace_bytes if down else ftq.workspace_bytes)(E, N, K, T, k, path)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev) if need else None
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    n_marks = 5 if down else 4

    def step(marks=None):
        if marks:
            marks[0].record()
        ftq.quantize_q8_1(x, out=aq)
        if marks:
            marks[1].record()
        ftq.moe_route(ids_d, E, ws, path)
        if marks:
            marks[2].record()
        matmul()
        if marks:
            marks[3].record()
        if down:
            ftq.combine_topk(out, gates_d, out=comb)
            if marks:
                marks[4].record()

    def matmul():
        if wt != 2:
            ftq.moe_gguf(wq, wt, aq, ids_d, E, N, K, per_pair=down, path=path, out=out, workspace=ws)
        elif down:
            ftq.moe_pairs_routed(wq, aq, ids_d, E, N, K, out, ws, path)
        elif fused:
            ftq.moe_act_routed(wq, aq, ids_d, E, N, K, act_kind, out, ws, path)
        else:
            ftq.moe_routed(wq, aq, ids_d, E, N, K, out, ws, path)

    steps = 3 if args.mode == "profile" else args.steps
    warmup = 2 if args.mode == "profile" else args.warmup
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Per-stage marks on eager steps (HIP events between the stages).  At decode
    # sizes a stage can take less GPU time than the host takes to submit the
    # next call, so these include submission gaps there; the step time and the
    # dominant kernel's time below come from graph replays, which keep the GPU
    # busy.
    marks = [[ev() for _ in range(n_marks)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(marks[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eager_ms_per_step = (t1 - t0) * 1e3 / steps
    q_ms = statistics.mean(m[0].elapsed_time(m[1]) for m in marks)
    r_ms = statistics.mean(m[1].elapsed_time(m[2]) for m in marks)
    mm_eager_ms = statistics.mean(m[2].elapsed_time(m[3]) for m in marks)
    cb_ms = statistics.mean(m[3].elapsed_time(m[4]) for m in marks) if down else None
    ref_out = (comb if down else out).clone()

    if args.mode == "profile":
        # plain copy of known size for counter calibration: 1 GiB read, 1 GiB written
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "profile", "ms_per_step": eager_ms_per_step, "matmul_ms": mm_eager_ms, "path": path}))
        return

    # One step captured as a HIP graph (every libftq call is capturable; the
    # library allocates and synchronises nothing), checked bit for bit against
    # the eager step, then replayed for the timed region.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        step()
    (comb if down else out).zero_()
    torch.cuda.synchronize()
    g_step.replay()
    torch.cuda.synchronize()
    if not torch.equal(comb if down else out, ref_out):
        print("bench.py: the graph-replayed step differs from the eager step", file=sys.stderr)
        sys.exit(1)

    # the same number of steps as graph replays (the host submits one graph
    # per step, so decode-size steps are no longer bound by per-call submission)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g_step.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    graph_ms_per_step = (t1 - t0) * 1e3 / steps
    ms_per_step = eager_ms_per_step
    # per-step GPU time of the timed eager steps (HIP events at the step's ends)
    warm_steps = [m[0].elapsed_time(m[-1]) for m in marks]
    # cold steps: each after a 1 GiB write, which leaves none of the step's
    # inputs in the L2s or the last-level cache
    scrub = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    cold_steps = _cold_times(step, scrub, args.cold_steps) if args.cold_steps > 0 else None

    # ---- the dominant kernel's duration ---------------------------------------
    # A call of 0.2 ms or more keeps the GPU behind the host, so the HIP events
    # between the stages of the eager steps bracket the kernel itself.  Shorter
    # calls take less GPU time than the host needs to submit the next one, so
    # they are timed with HIP events around a graph of R calls on the stream
    # they run on (per call); this agrees with the kernel trace, where the eager
    # marks would include submission gaps.
    R = 20
    kernel_from_graph = mm_eager_ms < 0.2
    mm_graph_ms = None
    if kernel_from_graph:
        g_mm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_mm):
            for _ in range(R):
                matmul()
        torch.cuda.synchronize()
        per_call = []
        for i in range(5):
            a, b = ev(), ev()
            a.record()
            g_mm.replay()
            b.record()
            torch.cuda.synchronize()
            per_call.append(a.elapsed_time(b) / R)
        mm_graph_ms = statistics.median(per_call)
    mm_ms = mm_graph_ms if kernel_from_graph else mm_eager_ms
    how = ("HIP events around a graph replay of 20 calls, per call" if kernel_from_graph
           else "HIP events between the stages of the timed eager steps, mean")

    # ---- roofline of the dominant kernel ------------------------------------
    pairs = T * k
    ops = 2.0 * pairs * N * K
    alg_bytes = _algorithmic_bytes(E, N, K, T, k, ids, act_rows, out_cols, W_BLOCK_BYTES[wt])
    kern_s = mm_ms / 1e3
    tops = ops / kern_s / 1e12
    gbs = alg_bytes / kern_s / 1e9
    traffic = None
    tf = traffic_file("moe_grouped_kernel" if path == ftq.PATH_GROUPED else "moe_gemv_kernel", args.workload, T)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("lib_sha256") == _lib_hash() and rec.get("T") == T:
            traffic = rec.get("bytes_per_launch")
    if path == ftq.PATH_GROUPED:
        roofline = {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                    "frac": round(tops / INT8_PEAK_TOPS, 4), "traffic": traffic,
                    "kernel": "moe_grouped_kernel (int8 MFMA block products, fp32 scale-accumulate)",
                    "kernel_ms": round(mm_ms, 4),
                    "kernel_ms_covers": "one routed matmul call: moe_grouped_kernel; " + how,
                    "frac_of_f16_peak": round(tops / F16_PEAK_TFLOPS, 4),
                    "ops_per_launch": ops, "alg_bytes_per_launch": alg_bytes,
                    "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "moe_gemv_kernel", "kernel_ms": round(mm_ms, 4),
                    "kernel_ms_covers": "one routed matmul call: moe_gemv_kernel; " + how,
                    "alg_bytes_per_launch": alg_bytes, "ops_per_launch": ops}

    # ---- decode records: the GEMV at Mixtral decode shapes -------------------
    decode = None
    if not args.no_decode:
        decode = [decode_record(name, t, scrub) for name, t in DECODE]
    sweep = None
    if not args.no_sweep and args.workload == "page1" and args.wtype == "q4_0" and T == DEFAULT_T:
        sweep = sweep_record(scrub)

    # ---- CPU oracle on a bounded sample of the same workload ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        ts = min(args.cpu_sample_tokens, T)
        # weight preparation: not part of a step
        ow = oracle.quantize_q4_0(w32).reshape(-1) if wt == 2 else wq.cpu().numpy().reshape(-1)
        c0 = time.perf_counter()
        if wt != 2:
            oa = oracle.quantize_q8_1(x32[:ts * k] if down else x32[:ts]).reshape(-1)
            oracle.moe_w(wt, ow, oa, np.ascontiguousarray(ids[:ts]), E, N, K, ts, k, per_pair=down)
        elif down:
            oa = oracle.quantize_q8_1(x32[:ts * k]).reshape(-1)
            y = oracle.moe(ow, oa, np.ascontiguousarray(ids[:ts]), E, N, K, ts, k, per_pair=True)
            oracle.combine_topk(y, gates[:ts])
        elif fused:
            oa = oracle.quantize_q8_1(x32[:ts]).reshape(-1)
            y = oracle.moe(ow, oa, np.ascontiguousarray(ids[:ts]), E, N, K, ts, k)
            oracle.act_and_mul(y, act_kind)
        else:
            oa = oracle.quantize_q8_1(x32[:ts]).reshape(-1)
            oracle.moe(ow, oa, np.ascontiguousarray(ids[:ts]), E, N, K, ts, k)
        c1 = time.perf_counter()
        cpu = {"value": round((c1 - c0) * 1e3 * T / ts, 1), "unit": "ms", "cores": oracle.num_threads(),
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"Q8_1 quantisation + matmul{' + combine' if down else (' + activation' if fused else '')} "
                         f"of the first {ts} of {T} "
                         f"tokens ({ts * k} of {pairs} pairs), "
                         f"{(c1 - c0):.1f} s measured, scaled by {T}/{ts} to one step"}

    result = {
        "metric": METRIC,
        "value": round(ms_per_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(ms_per_step / PAGES_MS_T8191, 6) if args.workload == "page1" and T == DEFAULT_T else None,
        "dtype": (f"{args.wtype} x q8_1 (exact integer block dots on int8 MFMA, fp32 scale-accumulate)" if path == ftq.PATH_GROUPED
                  else f"{args.wtype} x q8_1 (int8 dot4 block dots, fp32 scale-accumulate)"),
        "data": "synthetic",
        "config": dict(wl, T=T, pairs=pairs, path={1: "gemv", 2: "grouped"}[path], wtype=args.wtype),
        "timing": "value: wall clock over the timed steps issued eagerly; graph_ms_per_step: the same number of "
                  "steps as replays of one captured step graph (bit-identical output checked); breakdown: HIP events "
                  "between the stages of the eager steps (below 0.2 ms a stage includes host submission gaps), "
                  "matmul as roofline.kernel_ms_covers says",
        "graph_ms_per_step": round(graph_ms_per_step, 4),
        "step_ms": {"warm": _stats(warm_steps), "cold": _stats(cold_steps) if cold_steps else None,
                    "how": "HIP events at the ends of each step; warm: the timed eager steps; cold: each step right "
                           "after a 1 GiB write (no input left in the L2s or the last-level cache)"},
        "breakdown_ms": dict({"quantize_q8_1": round(q_ms, 4), "route": round(r_ms, 4), "matmul": round(mm_ms, 4),
                              "matmul_eager_marks": round(mm_eager_ms, 4),
                              "matmul_graph_per_call": round(mm_graph_ms, 4) if mm_graph_ms is not None else None},
                             **({"combine_topk": round(cb_ms, 4)} if down else {})),
        "throughput": dict({"tokens_per_s": round(T / (ms_per_step / 1e3), 1), "matmul_TOPS": round(tops, 2),
                            "matmul_alg_GBps": round(gbs, 1)},
                           # combine: reads y [T*k, N] and the gates, writes [T, N] (fp32)
                           **({"combine_alg_GBps": round((4 * T * k * N + 4 * T * k + 4 * T * N) / (cb_ms / 1e3) / 1e9, 1)}
                              if down else {})),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode": decode,
        "sweep": sweep,
        "host_cpu": cpu_model(),
        "lib_sha256": _lib_hash()[:16],
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
