#!/usr/bin/env python3
"""Throughput of the dense GEMM hot path on one MI355X.

A step is one pass over the two workloads the headline metric names, each a
full call of the library (plan, tile schedule, HBM->LDS staging, MFMA inner
product, alpha/beta epilogue):

  * fp32 SGEMM, row-major NN, M=N=8192, K=4096, alpha=1, beta=0, N(0,1) inputs;
  * fp16-input HGEMM, TN, M=N=K=4096, fp32 accumulate, fp16 C, N(0,1)/sqrt(K).

Inputs are seeded synthetic matrices, resident in HBM before timing starts.
``value`` is the whole step's throughput, 2*M*N*K summed over both GEMMs per
second, in TFLOPS.  The JSON line also carries each part's TFLOPS and its
fraction of MI355X's dense peak for its dtype, the roofline of the dominant
kernel (its average launch time from HIP events recorded on the launch
stream) and the CPU oracle timed on a bounded sample of the same step.

After the timed steps (outside the timed region): each part is timed again
with cold caches (a 512 MiB write before every launch, events around the
GEMM alone); the GPU clock (rocm-smi) and socket power (amd-smi) are read
while each part alone runs untimed; and a cache-blocked CPU GEMM (cpu_gemm/, fp32 accumulation, all
cores) runs the whole step as a second CPU baseline.  A workload whose tile
grid leaves CUs idle runs through the split-K entry point with the
workspace the planner asks for.  The fp32 part is also timed through
gemm_f32_split16 (fp32 accuracy from split fp16 inputs on the fp16 matrix
cores) and reported as "fp32_via_split_fp16", outside ``value``.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--cold-steps N] [--no-clocks] [--split16-steps N]
                       [--workload NAME ...] [--table] [--cpu-table]
"""
from __future__ import annotations

import argparse
import subprocess
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gemm_inputs as gi  # noqa: E402

METRIC = "GEMM TFLOPS & % of peak: fp32 8192×8192×4096, fp16 4096³ (1 MI355X)"
STEP = ("fp32_nn_8192x8192x4096", "fp16_tn_4096")
# MI355X dense peaks (TFLOP/s) per input type, and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}
HBM_GBPS = 8000.0
# The pages' own numbers for these workloads (RTX 4090; context only).
PAGES_CONTEXT = {
    "fp32_nn_8192x8192x4096": "RTX 4090: 41.9 TFLOPS hand-written (dbuf), 48.7-51.2 cuBLAS",
    "fp16_tn_4096": "RTX 4090: 148.5 TFLOPS (mma + smem swizzle, fp16 acc), 204 (warp-specialised)",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops(w):
    return 2.0 * w["M"] * w["N"] * w["K"]


def min_bytes(w):
    """Compulsory HBM traffic: read A, B (and C when beta != 0), write C."""
    es = 4 if w["in_dtype"] == "f32" else 2
    ec = 4 if w["c_dtype"] == "f32" else 2
    M, N, K = w["M"], w["N"], w["K"]
    return M * K * es + K * N * es + (M * N * ec if w["beta"] != 0 else 0) + M * N * ec


def load_traffic(config_name, workload):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(workload)
    from dense_gemm_12_amd.srchash import kernel_src_hash
    if not rec or rec.get("config") != config_name or rec.get("src_hash") != kernel_src_hash():
        return None
    return rec.get("l2_miss_bytes_per_launch")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(parts, target_s):
    """The oracle (as it stands) on a row slab of every part of the step."""
    import oracle
    threads = oracle.default_threads()
    total_flops, total_s, desc = 0.0, 0.0, []
    per_part = target_s / len(parts)
    for name, (A, B, C) in parts:
        w = gi.WORKLOADS[name]
        kw = dict(a_dtype=w["in_dtype"], trans_a=w["ta"], trans_b=w["tb"], alpha=w["alpha"],
                  beta=w["beta"], c_dtype=w["c_dtype"], M=w["M"], N=w["N"], K=w["K"])
        bits = lambda t: None if t is None else gi.as_numpy_bits(t)
        An, Bn, Cn = bits(A), bits(B), bits(C)
        # size the slab from two trial slabs (fixed cost + cost per row)
        pts = []
        rows = max(threads, 8)
        while True:
            n = min(rows, w["M"])
            t0 = time.perf_counter()
            oracle.gemm(An, Bn, C=Cn, rows=(0, n), threads=threads, **kw)
            pts.append((n, time.perf_counter() - t0))
            if (len(pts) >= 2 and pts[-1][1] > per_part / 10) or n >= w["M"]:
                break
            rows *= 4
        (n0, t0_), (n1, t1_) = (pts[-2] if len(pts) > 1 else (0, 0.0)), pts[-1]
        per_row = (t1_ - t0_) / max(n1 - n0, 1)
        if per_row <= 0:
            per_row = t1_ / max(n1, 1)
        fixed = max(t1_ - n1 * per_row, 0.0)
        rows = int(min(w["M"], max(1, (per_part - fixed) / per_row)))
        t0 = time.perf_counter()
        oracle.gemm(An, Bn, C=Cn, rows=(0, rows), threads=threads, **kw)
        dt = time.perf_counter() - t0
        f = 2.0 * rows * w["N"] * w["K"]
        total_flops += f
        total_s += dt
        desc.append(f"{name}: rows 0..{rows} of {w['M']} ({f / 1e9:.1f} GFLOP, {dt:.1f} s)")
    return {"value": total_flops / total_s / 1e12, "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "sample": "; ".join(desc) + "; fp64 triple loop, threads over rows",
            "seconds": round(total_s, 2), "cpu": cpu_model()}


def cpu_blocked(parts):
    """The blocked CPU GEMM (cpu_gemm/, fp32 accumulation, all cores) on every
    part of the step, whole problems."""
    import cpu_gemm
    threads = len(os.sched_getaffinity(0))
    cpu_gemm.load()
    total_flops, total_s, desc = 0.0, 0.0, []
    for name, (A, B, C) in parts:
        w = gi.WORKLOADS[name]
        An, Bn = gi.as_numpy_bits(A), gi.as_numpy_bits(B)
        Cn = None if C is None else C.float().numpy()
        t0 = time.perf_counter()
        cpu_gemm.gemm_rows(An, Bn, in_dtype=w["in_dtype"], ta=w["ta"], tb=w["tb"], M=w["M"], N=w["N"],
                           K=w["K"], alpha=w["alpha"], beta=w["beta"], Cin=Cn, threads=threads)
        dt = time.perf_counter() - t0
        total_flops += flops(w)
        total_s += dt
        desc.append(f"{name}: whole problem, {dt:.2f} s")
    return {"value": total_flops / total_s / 1e12, "unit": "TFLOPS", "cores": threads,
            "kind": "blocked", "sample": "; ".join(desc) + "; cache-blocked, packed, fp32 accumulate, "
            "gcc -O3 -march=native, threads over column stripes", "seconds": round(total_s, 2),
            "cpu": cpu_gemm.cpu_model()}


def _mhz(v):
    """'(2106Mhz)' -> 2106.0 (None if not a clock reading)."""
    import re
    m = re.search(r"(\d+(?:\.\d+)?)\s*Mhz", str(v), re.I)
    return float(m.group(1)) if m else None


def read_clocks():
    """GPU clocks and power from rocm-smi (None where it cannot say)."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True,
                           text=True, timeout=20)
        data = json.loads(r.stdout)
    except Exception:
        return None
    card = next((v for k, v in data.items() if k.startswith("card")), None)
    if not isinstance(card, dict):
        return None
    out = {}
    for k, v in card.items():
        key = k.lower()
        if key.startswith(("sclk", "mclk", "fclk", "socclk")) or "power" in key:
            out[k] = v
    w = read_socket_power()
    if w is not None:
        out["socket_power_w"] = w
    return out or None


def read_socket_power():
    """Socket power in W from amd-smi (rocm-smi reports none on this
    device); None where it cannot say.  The value is refreshed about once a
    second."""
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--json"], capture_output=True, text=True,
                           timeout=20)
        data = json.loads(r.stdout)
        gpus = data["gpu_data"] if isinstance(data, dict) else data
        v = gpus[0]["power"]["socket_power"]
        return float(v["value"] if isinstance(v, dict) else v)
    except Exception:
        return None


def workload_table(mg, torch, dev, names):
    """Per-launch time of each workload through the planner (through gemm_ex
    with a workspace where it would split or repack): warm (median of three
    runs of back-to-back launches) and cold (median launch after a 512 MiB
    buffer is overwritten)."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    codes = mg.DTYPE_CODES
    print("| workload | planner's kernel | warm µs | cold µs | TFLOPS (warm) | % of MFMA peak | "
          "min bytes / warm time |")
    print("|---|---|---|---|---|---|---|")
    for name in names:
        w = gi.WORKLOADS[name]
        A, B, C = gi.workload_inputs(name)
        A, B = A.to(dev), B.to(dev)
        C = (C.to(dev) if C is not None else
             torch.zeros((w["M"], w["N"]), dtype=gi.DTYPES[w["c_dtype"]], device=dev))
        key = (w["in_dtype"], w["c_dtype"], int(w["ta"]), int(w["tb"]), w["M"], w["N"], w["K"])
        wsb = mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], *key[2:], A.stride(0), B.stride(0))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
        cfg = (mg.chosen_config_ws(*key, A.stride(0), B.stride(0)) if ws is not None else mg.chosen_config(*key))
        kname = f"`{mg.config_name(w['in_dtype'], cfg)}`" + (" (gemm_ex)" if ws is not None else "")

        def call():
            mg.gemm(A, B, C, alpha=w["alpha"], beta=w["beta"], trans_a=w["ta"], trans_b=w["tb"], workspace=ws)

        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        reps = max(20, int(100.0 / max(e0.elapsed_time(e1), 1e-3)))
        trials = []
        for _ in range(3):
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            trials.append(e0.elapsed_time(e1) / reps * 1e3)
        warm = statistics.median(trials)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(reps, 40))]
        for a, b in ev:
            flush.zero_()
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        cold = statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3
        tf = flops(w) / warm / 1e6
        tbs = min_bytes(w) / warm / 1e6
        print(f"| {name} | {kname} | {warm:.1f} | {cold:.1f} | {tf:.1f} | {100 * tf / PEAK_TFLOPS[w['in_dtype']]:.1f} % | "
              f"{tbs:.2f} TB/s ({100 * tbs / 8:.0f} % of 8) |", flush=True)
        del A, B, C, ws
        torch.cuda.empty_cache()


def cpu_table(mg, torch, dev, names, budget_s=60.0):
    """Per-workload CPU baselines beside the GPU time: the oracle on the whole
    problem when a trial slab predicts at most ``budget_s`` seconds, else on a
    row slab scaled by M / rows (marked extrapolated; the work is linear in
    M); the blocked CPU GEMM likewise; GPU per-launch time (warm, median of
    three runs of back-to-back launches through the planner, as ``--table``)."""
    import oracle
    import cpu_gemm
    threads = oracle.default_threads()
    model = cpu_model()
    codes = mg.DTYPE_CODES
    rows_out = []
    print(f"CPU: {model}, {threads} threads", flush=True)
    print("| workload | GFLOP | GPU µs (warm) | oracle: rows timed | oracle s (full) | oracle GFLOP/s | "
          "GPU speed-up vs oracle | blocked: rows timed | blocked s (full) | blocked GFLOP/s | "
          "GPU speed-up vs blocked |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for name in names:
        w = gi.WORKLOADS[name]
        A, B, C = gi.workload_inputs(name)
        M, N, K = w["M"], w["N"], w["K"]
        fl = flops(w)
        # GPU: the planner's launch (through gemm_ex when it asks for a workspace)
        Ad, Bd = A.to(dev), B.to(dev)
        Cd = C.to(dev) if C is not None else torch.zeros((M, N), dtype=gi.DTYPES[w["c_dtype"]], device=dev)
        wsb = mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]), M, N, K,
                                Ad.stride(0), Bd.stride(0))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
        call = lambda: mg.gemm(Ad, Bd, Cd, alpha=w["alpha"], beta=w["beta"], trans_a=w["ta"], trans_b=w["tb"],
                               workspace=ws)
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        reps = max(20, int(100.0 / max(e0.elapsed_time(e1), 1e-3)))
        tr = []
        for _ in range(3):
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            tr.append(e0.elapsed_time(e1) / reps * 1e-3)
        gpu_s = statistics.median(tr)
        del Ad, Bd, Cd, ws
        torch.cuda.empty_cache()
        bits = lambda t: None if t is None else gi.as_numpy_bits(t)
        An, Bn, Cn = bits(A), bits(B), bits(C)
        kw = dict(a_dtype=w["in_dtype"], trans_a=w["ta"], trans_b=w["tb"], alpha=w["alpha"], beta=w["beta"],
                  c_dtype=w["c_dtype"], M=M, N=N, K=K)

        def timed(fn, r):
            t0 = time.perf_counter()
            fn(r)
            return time.perf_counter() - t0

        def measure(fn):
            # trial slab, then the whole problem or a slab of about budget_s / 4
            trial = min(M, max(threads, 16))
            t_trial = timed(fn, trial)
            est_full = t_trial * M / trial
            if est_full <= budget_s:
                return M, timed(fn, M), False
            r = int(min(M, max(trial, M * (budget_s / 4) / est_full)))
            return r, timed(fn, r) * M / r, True

        o_rows, o_s, o_ext = measure(lambda r: oracle.gemm(An, Bn, C=Cn, rows=(0, r), threads=threads, **kw))
        Cf = None if C is None else C.float().numpy()
        b_rows, b_s, b_ext = measure(lambda r: cpu_gemm.gemm_rows(
            An, Bn, in_dtype=w["in_dtype"], ta=w["ta"], tb=w["tb"], M=M, N=N, K=K, alpha=w["alpha"],
            beta=w["beta"], Cin=Cf, rows=(0, r), threads=threads))
        rec = {"workload": name, "gflop": fl / 1e9, "gpu_us": gpu_s * 1e6, "oracle_rows": o_rows,
               "oracle_s": o_s, "oracle_extrapolated": o_ext, "blocked_rows": b_rows, "blocked_s": b_s,
               "blocked_extrapolated": b_ext, "cores": threads, "cpu": model}
        rows_out.append(rec)
        mark = lambda e: " (extrapolated)" if e else ""
        print(f"| {name} | {fl / 1e9:.3g} | {gpu_s * 1e6:.1f} | {o_rows} of {M} | {o_s:.3g}{mark(o_ext)} | "
              f"{fl / o_s / 1e9:.1f} | {o_s / gpu_s:.3g}x | {b_rows} of {M} | {b_s:.3g}{mark(b_ext)} | "
              f"{fl / b_s / 1e9:.1f} | {b_s / gpu_s:.3g}x |", flush=True)
    print(json.dumps({"cpu_table": rows_out}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--workload", nargs="*", default=None,
                    help=f"named workloads instead of the metric's step {STEP}")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps with a 512 MiB cache scrub before each launch (0: skip)")
    ap.add_argument("--no-clocks", action="store_true", help="skip the clock and power readings")
    ap.add_argument("--table", action="store_true",
                    help="instead of the step: time every named workload (or --workload) through the "
                         "planner, warm and after a cache scrub, and print a markdown table")
    ap.add_argument("--cpu-table", action="store_true",
                    help="instead of the step: every named workload (or --workload) on the GPU and on the host "
                         "(oracle and blocked CPU GEMM, whole problem or an extrapolated slab), as a markdown "
                         "table")
    ap.add_argument("--split16-steps", type=int, default=10,
                    help="launches of the fp32 part through split fp16 inputs, reported beside the "
                         "step (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the GEMM is not sharded "
              "across GPUs in this library.", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch
    import dense_gemm_12_amd as mg
    mg.load()
    dev = torch.device("cuda:0")
    if args.table:
        workload_table(mg, torch, dev, tuple(args.workload) if args.workload else tuple(gi.WORKLOADS))
        return
    if args.cpu_table:
        cpu_table(mg, torch, dev, tuple(args.workload) if args.workload else tuple(gi.WORKLOADS))
        return
    names = tuple(args.workload) if args.workload else STEP

    parts_host, parts_dev, calls = [], [], []
    for name in names:
        w = gi.WORKLOADS[name]
        log(f"inputs {name}")
        A, B, C = gi.workload_inputs(name)
        parts_host.append((name, (A, B, C)))
        Ad, Bd = A.to(dev), B.to(dev)
        Cd = (C.to(dev) if C is not None else
              torch.empty((w["M"], w["N"]), dtype=gi.DTYPES[w["c_dtype"]], device=dev))
        parts_dev.append((Ad, Bd, Cd))
        # problems whose tile grid leaves CUs idle run split-K with a workspace
        codes = mg.DTYPE_CODES
        wsb = mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]),
                                w["M"], w["N"], w["K"], Ad.stride(0), Bd.stride(0))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
        calls.append((name, w, Ad, Bd, Cd, ws))

    stream = torch.cuda.current_stream(dev)

    def launch(w, Ad, Bd, Cd, ws):
        mg.gemm(Ad, Bd, Cd, alpha=w["alpha"], beta=w["beta"], trans_a=w["ta"], trans_b=w["tb"],
                stream=stream, workspace=ws)

    def step(evs=None):
        for i, (name, w, Ad, Bd, Cd, ws) in enumerate(calls):
            if evs is not None:
                evs[i][0].record(stream)
            launch(w, Ad, Bd, Cd, ws)
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in calls]
              for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    cold_ms = None
    if args.cold_steps > 0:
        # Cold caches: a 512 MiB write (twice the Infinity Cache) before every
        # launch evicts A, B and C; the events bracket the GEMM alone.
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in calls]
               for _ in range(args.cold_steps)]
        log(f"timing {args.cold_steps} cold-cache steps")
        for k in range(args.cold_steps):
            for i, (name, w, Ad, Bd, Cd, ws) in enumerate(calls):
                scrub.fill_(k & 0xff)
                cev[k][i][0].record(stream)
                launch(w, Ad, Bd, Cd, ws)
                cev[k][i][1].record(stream)
        torch.cuda.synchronize()
        cold_ms = [sum(cev[k][i][0].elapsed_time(cev[k][i][1]) for k in range(args.cold_steps)) /
                   args.cold_steps for i in range(len(calls))]
        del scrub
    # Per part, outside the timed region: five trials of back-to-back
    # launches (each trial at least ~100 ms of GPU time), per-launch median
    # and minimum, with HIP events on the launch stream.
    trials = []
    for i, (name, w, Ad, Bd, Cd, ws) in enumerate(calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch(w, Ad, Bd, Cd, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        reps = max(20, int(100.0 / max(e0.elapsed_time(e1), 1e-3)) + 1)
        per = []
        for _ in range(5):
            e0.record(stream)
            for _ in range(reps):
                launch(w, Ad, Bd, Cd, ws)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / reps * 1e3)
        trials.append({"trials": 5, "launches_per_trial": reps, "us_median": round(statistics.median(per), 2),
                       "us_min": round(min(per), 2)})

    clocks = None
    part_clocks = [None] * len(calls)
    if not args.no_clocks:
        # Clocks and socket power under each part's own load: rocm-smi and
        # amd-smi are read for about 3 s while that part alone runs back to
        # back, and only readings from the last 1.5 s are kept (the power
        # figure is refreshed about once a second), so each reading describes
        # the kernel it is reported with.
        import threading
        for i, (name, w, Ad, Bd, Cd, ws) in enumerate(calls):
            holder = {"samples": []}
            t_start = time.perf_counter()

            def sampler():
                while time.perf_counter() - t_start < 3.0:
                    c = read_clocks()
                    if c and time.perf_counter() - t_start >= 1.5:
                        holder["samples"].append(c)
                    elif not c:
                        time.sleep(0.2)

            th = threading.Thread(target=sampler)
            th.start()
            t_end = time.perf_counter() + 30.0
            while th.is_alive() and time.perf_counter() < t_end:
                for _ in range(10):
                    launch(w, Ad, Bd, Cd, ws)
                torch.cuda.synchronize()
            th.join()
            sclk = [mhz for c in holder["samples"] for k, v in c.items()
                    if k.lower().startswith("sclk clock speed") and (mhz := _mhz(v)) is not None]
            pw = [c["socket_power_w"] for c in holder["samples"] if c.get("socket_power_w") is not None]
            part_clocks[i] = {"sclk_mhz_samples": sclk,
                              "sclk_mhz_median": statistics.median(sclk) if sclk else None,
                              "socket_power_w_median": statistics.median(pw) if pw else None,
                              "readings": holder["samples"][-1] if holder["samples"] else None}
        clocks = {calls[i][0]: part_clocks[i] for i in range(len(calls))}

    split16 = None
    f32_calls = [c for c in calls if c[1]["in_dtype"] == "f32"]
    if args.split16_steps > 0 and f32_calls:
        # The fp32 part again through gemm_f32_split16 (fp32 accuracy from
        # fp16 matrix cores); reported beside the step, not in its value.
        name, w, Ad, Bd, Cd, _ws = f32_calls[0]
        wsb = mg.split16_workspace_size(w["M"], w["N"], w["K"])
        ws16 = torch.empty(wsb, dtype=torch.uint8, device=dev)
        f = lambda: mg.gemm(Ad, Bd, Cd, alpha=w["alpha"], beta=w["beta"], trans_a=w["ta"],
                            trans_b=w["tb"], stream=stream, split16=True, workspace=ws16)
        for _ in range(2):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.split16_steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.split16_steps
        kp = (w["K"] + 63) // 64 * 64
        mfma_flops = 2.0 * w["M"] * w["N"] * 3 * kp
        split16 = {"workload": name, "entry": "gemm_f32_split16", "us_per_launch": round(ms * 1e3, 2),
                   "tflops_algorithmic": round(flops(w) / (ms * 1e-3) / 1e12, 2),
                   "fp16_mfma_flops_per_launch": mfma_flops,
                   "fp16_mfma_tflops": round(mfma_flops / (ms * 1e-3) / 1e12, 2),
                   "frac_of_fp16_peak": round(mfma_flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["f16"], 4),
                   "workspace_bytes": wsb,
                   "note": "fp32 result within 1e-5*|a_i||b_j| from split fp16 inputs; includes the "
                           "split/scale passes; not part of value"}
        del ws16

    step_flops = sum(flops(w) for _, w, *_ in calls)
    value = args.steps * step_flops / elapsed / 1e12
    parts = []
    for i, (name, w, *_r) in enumerate(calls):
        ms = sum(events[k][i][0].elapsed_time(events[k][i][1]) for k in range(args.steps)) / args.steps
        if calls[i][5] is not None:  # the workspace path (split-K / repacked operands)
            cfg = mg.chosen_config_ws(w["in_dtype"], w["c_dtype"], int(w["ta"]), int(w["tb"]), w["M"],
                                      w["N"], w["K"], calls[i][2].stride(0), calls[i][3].stride(0))
        else:
            cfg = mg.chosen_config(w["in_dtype"], w["c_dtype"], int(w["ta"]), int(w["tb"]), w["M"],
                                   w["N"], w["K"])
        tf = flops(w) / (ms * 1e-3) / 1e12
        parts.append({"workload": name, "kernel": mg.config_name(w["in_dtype"], cfg),
                      "us_per_launch": round(ms * 1e3, 2), "tflops": round(tf, 2),
                      "peak_tflops": PEAK_TFLOPS[w["in_dtype"]],
                      "frac_of_peak": round(tf / PEAK_TFLOPS[w["in_dtype"]], 4),
                      "min_hbm_bytes": min_bytes(w),
                      "split_k_workspace_bytes": 0 if calls[i][5] is None else calls[i][5].numel(),
                      "pages_context": PAGES_CONTEXT.get(name)})
        parts[-1]["launch_trials"] = trials[i]
        if part_clocks[i] is not None:
            parts[-1]["sclk_mhz_under_own_load"] = part_clocks[i]["sclk_mhz_median"]
            parts[-1]["socket_power_w_under_own_load"] = part_clocks[i]["socket_power_w_median"]
        if cold_ms is not None:
            parts[-1]["us_per_launch_cold"] = round(cold_ms[i] * 1e3, 2)
            parts[-1]["tflops_cold"] = round(flops(w) / (cold_ms[i] * 1e-3) / 1e12, 2)
            parts[-1]["hbm_gbps_cold_min_bytes"] = round(min_bytes(w) / (cold_ms[i] * 1e-3) / 1e9, 1)
    dom = max(range(len(parts)), key=lambda i: parts[i]["us_per_launch"])
    d, dw = parts[dom], calls[dom][1]
    traffic = load_traffic(d["kernel"], d["workload"])
    roofline = {"bound": "mfma", "achieved": d["tflops"], "peak": d["peak_tflops"],
                "unit": "TFLOP/s", "frac": d["frac_of_peak"], "traffic": traffic,
                "kernel": d["kernel"], "workload": d["workload"],
                "algorithmic_flops_per_launch": flops(dw)}
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "+".join(sorted({w["in_dtype"] for _, w, *_ in calls})),
        "data": "synthetic: seeded fp32 N(0,1) and fp16 N(0,1)/sqrt(K) matrices, resident in HBM",
        "config": {"workload": " + ".join(names), "parts": list(names)},
        "parts": parts, "roofline": roofline, "gpu_clocks_per_part": clocks,
        "fp32_via_split_fp16": split16,
    }
    if not args.no_cpu and rank == 0:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(parts_host, args.cpu_seconds)
        log("CPU blocked baseline")
        out["cpu_blocked"] = cpu_blocked(parts_host)
    if rank == 0:
        print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
