"""rocprofv3 harness: hardware counters of the GEMM kernels against MI355X's peaks.

Two modes:

``python -m dense_gemm_12_amd.rocprof_harness run --workload fp16_tn_4096 --out DIR``
    Runs one rocprofv3 pass per counter group (each group stays within the
    per-block limits of one pass), each over ``target`` below, then parses
    the CSV output and writes ``DIR/summary.json`` and ``DIR/summary.md``:
    MFMA utilisation, VALU busy (both from raw counters and, as a cross-check,
    from rocprofiler-sdk's own derived ``MfmaUtil`` / ``VALUBusy``), LDS
    bank-conflict rate, effective shader clock, L2-miss traffic (FETCH_SIZE /
    WRITE_SIZE calibrated against a plain copy of known size), the part of it
    addressed to DRAM (TCC_EA0_*_DRAM_32B; Infinity-Cache hits still count
    there) and achieved TFLOPS / GB/s against the peaks.

``python -m dense_gemm_12_amd.rocprof_harness target --workload NAME [--iters N] [--config C]``
    The program each pass profiles: uploads the workload's seeded inputs and
    runs the library's GEMM ``iters`` times; ``--workload copy`` instead runs a
    1 GiB device-to-device copy (the calibration kernel).

``python -m dense_gemm_12_amd.rocprof_harness collect DIR [DIR ...] [--profiles profiles]``
    Copies each run's summary into ``profiles/counters_<workload>.md`` and
    records its calibrated HBM traffic, kernel configuration and kernel
    source hash in ``profiles/traffic.json`` (the file the benchmark reads its
    ``traffic`` figure from, valid only while hash and configuration match).

The driver never touches the GPU itself; each pass is a fresh process started
directly by rocprofv3.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CUS, SIMDS = 256, 1024
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}
HBM_GBPS = 8000.0
COPY_BYTES = 1 << 30

# One rocprofv3 pass per group: <= 8 SQ, <= 4 TCC (FETCH_SIZE uses 3,
# WRITE_SIZE 2), <= 2 GRBM counters.
PASSES = {
    "fetch": ["FETCH_SIZE", "GRBM_GUI_ACTIVE"],
    "write": ["WRITE_SIZE", "GRBM_GUI_ACTIVE"],
    "dram": ["TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", "GRBM_GUI_ACTIVE"],
    "sq": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_LDS_BANK_CONFLICT",
           "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_BUSY_CU_CYCLES",
           "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"],
    # rocprofiler-sdk's derived metrics (counter_defs.yaml, gfx950):
    #   MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMD_NUM)
    #   VALUBusy = 100 * sum(SQ_ACTIVE_INST_VALU) / CU_NUM / max(GRBM_GUI_ACTIVE)
    "derived": ["MfmaUtil", "VALUBusy"],
}


def _target(args):
    sys.path.insert(0, ROOT)
    import torch
    import gemm_inputs as gi
    import dense_gemm_12_amd as mg
    dev = torch.device("cuda:0")
    if args.workload == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.iters):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy x{args.iters} done", flush=True)
        return
    w = gi.WORKLOADS[args.workload]
    A, B, C = gi.workload_inputs(args.workload)
    Ad, Bd = A.to(dev), B.to(dev)
    Cd = C.to(dev) if C is not None else torch.zeros((w["M"], w["N"]), dtype=gi.DTYPES[w["c_dtype"]],
                                                     device=dev)
    cfg = -1 if args.config is None else mg.config_id(w["in_dtype"], args.config)
    # the benchmark's launch configuration: gemm_ex with the planner's
    # workspace when it asks for one (split-K, repacking, stream-K)
    codes = mg.DTYPE_CODES
    wsb = mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]), w["M"], w["N"],
                            w["K"], Ad.stride(0), Bd.stride(0)) if cfg < 0 else 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    # warm-up launches first (not profiled: the counter passes select the
    # measured dispatches by iteration), so the measured ones run at the
    # clock and power state of sustained load
    for _ in range(args.warmup + args.iters):
        mg.gemm(Ad, Bd, Cd, alpha=w["alpha"], beta=w["beta"], trans_a=w["ta"], trans_b=w["tb"],
                config=cfg, workspace=ws)
    torch.cuda.synchronize()
    print(f"{args.workload} x{args.iters} done", flush=True)


def _read_counters(pass_dir):
    """{kernel name: {counter: [per-dispatch values]}} plus durations (ns)."""
    files = glob.glob(os.path.join(pass_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no counter_collection.csv under {pass_dir}")
    per = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                k = row["Kernel_Name"]
                d = per.setdefault(k, {"dispatch": {}})
                key = row.get("Dispatch_Id") or row.get("Correlation_Id")
                disp = d["dispatch"].setdefault(key, {})
                disp[row["Counter_Name"]] = disp.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
                for tk in ("Start_Timestamp", "End_Timestamp"):
                    if row.get(tk):
                        disp[tk] = float(row[tk])
    return per


def _last(per_kernel, n):
    """The kernel's last n dispatches (by dispatch id): the measured ones
    even if the profiler also counted warm-up dispatches."""
    if per_kernel is None:
        return None
    keys = sorted(per_kernel["dispatch"], key=lambda k: float(k) if k not in (None, "") else -1.0)
    return {"dispatch": {k: per_kernel["dispatch"][k] for k in keys[-n:]}}


def _avg(per_kernel, counter):
    vals = [d[counter] for d in per_kernel["dispatch"].values() if counter in d]
    return sum(vals) / len(vals) if vals else None


def _run_pass(name, counters, target_args, out, iterations=None):
    """One --pmc pass; iterations = (first, last): only those dispatches of
    the GEMM kernel (1-based, in launch order) get counters."""
    pdir = os.path.join(out, name)
    os.makedirs(pdir, exist_ok=True)
    sel = []
    if iterations is not None:
        sel = ["--kernel-include-regex", "gemm", "--kernel-iteration-range",
               f"[{iterations[0]}-{iterations[1]}]"]
    cmd = ["rocprofv3", "--pmc", *counters, *sel, "--output-format", "csv", "-d", pdir, "-o", name, "--",
           sys.executable, "-m", "dense_gemm_12_amd.rocprof_harness", "target", *target_args]
    print("pass:", " ".join(cmd), flush=True)
    t0 = time.time()
    r = subprocess.run(cmd, cwd="/tmp", env={**os.environ, "TMPDIR": "/tmp", "PYTHONPATH": ROOT},
                       timeout=300)
    print(f"pass {name}: rc={r.returncode} in {time.time() - t0:.1f}s", flush=True)
    # rocprofv3 may exit non-zero after a complete run; the CSV decides.
    return _read_counters(pdir)


def _run_trace(name, target_args, out):
    """Kernel durations (ns) from a kernel-trace run with no counters:
    {kernel name: [duration per dispatch, in launch order]}."""
    pdir = os.path.join(out, name)
    os.makedirs(pdir, exist_ok=True)
    cmd = ["rocprofv3", "--kernel-trace", "--output-format", "csv", "-d", pdir, "-o", name, "--",
           sys.executable, "-m", "dense_gemm_12_amd.rocprof_harness", "target", *target_args]
    print("pass:", " ".join(cmd), flush=True)
    t0 = time.time()
    r = subprocess.run(cmd, cwd="/tmp", env={**os.environ, "TMPDIR": "/tmp", "PYTHONPATH": ROOT},
                       timeout=300)
    print(f"pass {name}: rc={r.returncode} in {time.time() - t0:.1f}s", flush=True)
    return _read_trace(pdir)


def _read_trace(pdir):
    """{kernel name: [duration (ns) per dispatch, in launch order]} from the
    kernel_trace.csv files under pdir."""
    files = glob.glob(os.path.join(pdir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no kernel_trace.csv under {pdir}")
    per = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                per.setdefault(row["Kernel_Name"], []).append(
                    (float(row["Start_Timestamp"]), float(row["End_Timestamp"]) - float(row["Start_Timestamp"])))
    return {k: [d for _, d in sorted(v)] for k, v in per.items()}  # durations in launch order


def _pick(per, want):
    """The kernel whose name contains `want` with the most dispatches."""
    best = None
    for k, v in per.items():
        if want in k and (best is None or len(v["dispatch"]) > len(per[best]["dispatch"])):
            best = k
    return best


def run(args):
    sys.path.insert(0, ROOT)
    import gemm_inputs as gi
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    w = gi.WORKLOADS[args.workload]
    # about 1.5 s of warm-up launches (estimated at half the peak rate),
    # 20 to 30000 of them
    est_s = 2.0 * w["M"] * w["N"] * w["K"] / (0.5 * PEAK_TFLOPS[w["in_dtype"]] * 1e12)
    warm = int(min(30000, max(20, 1.5 / est_s))) if args.warmup < 0 else args.warmup
    tgt = ["--workload", args.workload, "--iters", str(args.iters), "--warmup", str(warm)]
    if args.config:
        tgt += ["--config", args.config]
    measured = (warm + 1, warm + args.iters)
    results = {}
    for name, counters in PASSES.items():
        results[name] = _run_pass(name, counters, tgt, out, iterations=measured)
    trace = _run_trace("trace", tgt, out)
    calib = {}
    for name in ("fetch", "write", "dram"):
        calib[name] = _run_pass("copy_" + name, PASSES[name], ["--workload", "copy", "--iters", "3"],
                                out)
    kname = _pick(results["sq"], "gemm")
    copy_k = max(calib["fetch"], key=lambda k: len(calib["fetch"][k]["dispatch"]))
    fetch_copy = _avg(calib["fetch"][copy_k], "FETCH_SIZE")
    write_copy = _avg(calib["write"][copy_k], "WRITE_SIZE")
    f_factor = COPY_BYTES / (fetch_copy * 1024) if fetch_copy else None
    w_factor = COPY_BYTES / (write_copy * 1024) if write_copy else None
    dcopy_k = max(calib["dram"], key=lambda k: len(calib["dram"][k]["dispatch"]))
    dram_rd_copy = _avg(calib["dram"][dcopy_k], "TCC_EA0_RDREQ_DRAM_32B_sum")
    dram_wr_copy = _avg(calib["dram"][dcopy_k], "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")

    w = gi.WORKLOADS[args.workload]
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    sq = _last(results["sq"][kname], args.iters)
    gui = _avg(sq, "GRBM_GUI_ACTIVE")
    mfma = _avg(sq, "SQ_VALU_MFMA_BUSY_CYCLES")
    valu = _avg(sq, "SQ_ACTIVE_INST_VALU")
    bank = _avg(sq, "SQ_LDS_BANK_CONFLICT")
    ldsact = _avg(sq, "SQ_LDS_IDX_ACTIVE")
    durs = [d["End_Timestamp"] - d["Start_Timestamp"] for d in sq["dispatch"].values()
            if "End_Timestamp" in d]
    dur_ns = sorted(durs)[len(durs) // 2] if durs else None
    tk = _pick({k: {"dispatch": dict(enumerate(v))} for k, v in trace.items()}, "gemm")
    tr = sorted(trace[tk][-args.iters:]) if tk else []  # the measured launches, after the warm-up
    trace_ns = tr[len(tr) // 2] if tr else None
    # GRBM_GUI_ACTIVE is reported per XCD and summed over the 8 XCDs.
    gui_cycles = gui / 8 if gui else None
    fetch_kib = _avg(_last(results["fetch"][_pick(results["fetch"], "gemm")], args.iters), "FETCH_SIZE")
    write_kib = _avg(_last(results["write"][_pick(results["write"], "gemm")], args.iters), "WRITE_SIZE")
    dr = _last(results["dram"][_pick(results["dram"], "gemm")], args.iters)
    dram_rd = _avg(dr, "TCC_EA0_RDREQ_DRAM_32B_sum")
    dram_wr = _avg(dr, "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
    der = _last(results["derived"][_pick(results["derived"], "gemm")], args.iters)
    sdk_mfma = _avg(der, "MfmaUtil")
    sdk_valu = _avg(der, "VALUBusy")
    es = 4 if w["in_dtype"] == "f32" else 2
    ec = 4 if w["c_dtype"] == "f32" else 2
    min_bytes = (w["M"] * w["K"] + w["K"] * w["N"]) * es + w["M"] * w["N"] * ec * (2 if w["beta"] else 1)
    fetch_b = fetch_kib * 1024 * f_factor if (fetch_kib is not None and f_factor) else None
    write_b = write_kib * 1024 * w_factor if (write_kib is not None and w_factor) else None
    import dense_gemm_12_amd as mg
    from dense_gemm_12_amd.srchash import kernel_src_hash
    lib = mg.load()
    codes = mg.DTYPE_CODES
    lda = w["M"] if w["ta"] else w["K"]
    ldb = w["K"] if w["tb"] else w["N"]
    if mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]), w["M"], w["N"],
                         w["K"], lda, ldb):
        cfg_id = mg.chosen_config_ws(w["in_dtype"], w["c_dtype"], int(w["ta"]), int(w["tb"]), w["M"], w["N"],
                                     w["K"], lda, ldb)
    else:
        cfg_id = lib.mg_chosen_config(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]),
                                      w["M"], w["N"], w["K"])
    summary = {
        "workload": args.workload, "kernel": kname, "iters": args.iters,
        "config": args.config or mg.config_name(w["in_dtype"], cfg_id),
        "src_hash": kernel_src_hash(),
        "warmup_launches": warm,
        "dispatches": len(sq["dispatch"]),
        "kernel_ns_median": trace_ns,
        "kernel_ns_median_under_pmc": dur_ns,
        "gui_active_cycles": gui_cycles,
        # cycles counted in the counter pass over the measured launches'
        # duration in the kernel-trace pass
        "effective_clock_ghz": (gui_cycles / trace_ns) if (gui_cycles and trace_ns) else None,
        "mfma_util_pct": 100.0 * mfma / (gui_cycles * SIMDS) if (mfma and gui_cycles) else None,
        "valu_busy_pct": 100.0 * valu / CUS / gui_cycles if (valu and gui_cycles) else None,
        "lds_bank_conflict_per_access": bank / (ldsact - bank) if (ldsact and ldsact > bank) else None,
        "lds_bank_conflict_cycles_pct": 100.0 * bank / (gui_cycles * CUS) if (bank is not None and gui_cycles) else None,
        "sq_insts_mfma": _avg(sq, "SQ_INSTS_MFMA"), "sq_insts_lds": _avg(sq, "SQ_INSTS_LDS"),
        "sdk_MfmaUtil_pct": sdk_mfma, "sdk_VALUBusy_pct": sdk_valu,
        "fetch_kib_raw": fetch_kib, "write_kib_raw": write_kib,
        "copy_calibration": {"bytes_each_way": COPY_BYTES, "fetch_kib": fetch_copy,
                             "write_kib": write_copy, "fetch_factor": f_factor,
                             "write_factor": w_factor},
        "l2_miss_fetch_bytes": fetch_b, "l2_miss_write_bytes": write_b,
        "l2_miss_bytes_per_launch": (fetch_b + write_b) if (fetch_b is not None and write_b is not None) else None,
        "dram_32b_reads": dram_rd, "dram_32b_writes": dram_wr,
        "dram_copy_calibration": {"bytes_each_way": COPY_BYTES, "rd_32b": dram_rd_copy, "wr_32b": dram_wr_copy},
        "dram_read_bytes": dram_rd * 32 if dram_rd is not None else None,
        "dram_write_bytes": dram_wr * 32 if dram_wr is not None else None,
        "min_bytes_per_launch": min_bytes,
        "flops_per_launch": flops,
    }
    if trace_ns:
        summary["tflops"] = flops / trace_ns / 1e3
        summary["frac_of_peak"] = summary["tflops"] / PEAK_TFLOPS[w["in_dtype"]]
        if summary["l2_miss_bytes_per_launch"]:
            summary["l2_miss_gbps"] = summary["l2_miss_bytes_per_launch"] / trace_ns
        if dram_rd is not None and dram_wr is not None:
            summary["dram_gbps"] = (dram_rd + dram_wr) * 32 / trace_ns
            summary["dram_frac_of_hbm_peak"] = summary["dram_gbps"] / HBM_GBPS
    # The raw-counter derivations must agree with rocprofiler-sdk's own
    # (different passes, so a few per cent of run-to-run spread is allowed).
    for mine, sdk in (("mfma_util_pct", "sdk_MfmaUtil_pct"), ("valu_busy_pct", "sdk_VALUBusy_pct")):
        a, b = summary.get(mine), summary.get(sdk)
        summary[mine + "_agrees_with_sdk"] = (a is not None and b is not None and
                                              abs(a - b) <= 0.1 * max(abs(b), 1.0))
    with open(os.path.join(out, "summary.json"), "w") as f:
        json.dump(summary, f, indent=2)
    lines = [f"# Counters: {args.workload}", "", f"kernel: `{kname}`", "",
             "| metric | value |", "|---|---|"]
    for k, v in summary.items():
        if isinstance(v, dict):
            v = json.dumps(v)
        elif isinstance(v, float):
            v = f"{v:.4g}"
        lines.append(f"| {k} | {v} |")
    with open(os.path.join(out, "summary.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(summary, indent=2), flush=True)


def collect(dirs, profiles):
    path = os.path.join(profiles, "traffic.json")
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    for d in dirs:
        with open(os.path.join(d, "summary.json")) as f:
            s = json.load(f)
        w = s["workload"]
        cal = s["copy_calibration"]
        table[w] = {"config": s["config"], "src_hash": s["src_hash"],
                    "l2_miss_bytes_per_launch": s["l2_miss_bytes_per_launch"],
                    "l2_miss_fetch_bytes": s["l2_miss_fetch_bytes"],
                    "l2_miss_write_bytes": s["l2_miss_write_bytes"],
                    "dram_read_bytes": s.get("dram_read_bytes"), "dram_write_bytes": s.get("dram_write_bytes"),
                    "fetch_factor": cal["fetch_factor"], "write_factor": cal["write_factor"],
                    "source": f"profiles/counters_{w}.md"}
        with open(os.path.join(d, "summary.md")) as f:
            body = f.read().split("\n", 1)[1]
        cmd = (f"python3 -m dense_gemm_12_amd.rocprof_harness run --workload {w} --iters "
               f"{s.get('iters', 5)} --out $OUT/harness_{w}")
        text = (f"# Hardware counters: {w}\n\n"
                "Command ($OUT: any scratch directory; each counter group is one rocprofv3 --pmc pass over "
                "the workload, then one --kernel-trace pass without counters for the kernel's duration; "
                "each run first launches the GEMM unprofiled for about 1.5 s (warmup_launches) and counts "
                "only the measured launches after it (--kernel-iteration-range), so the figures describe "
                "sustained load, "
                "plus three passes over a 1 GiB copy for calibrating FETCH_SIZE, WRITE_SIZE and the DRAM "
                "request counters):\n\n"
                f"```\n{cmd}\n```\n\nKernel configuration `{s['config']}`, kernel source hash "
                f"`{s['src_hash']}`.\n{body}\n"
                f"Calibration: a {cal['bytes_each_way']} B device copy reads FETCH_SIZE = "
                f"{cal['fetch_kib']:.0f} KiB and WRITE_SIZE = {cal['write_kib']:.0f} KiB, so fetched "
                f"bytes = FETCH_SIZE x 1024 x {cal['fetch_factor']:.4f} and written bytes = WRITE_SIZE "
                f"x 1024 x {cal['write_factor']:.4f}.\n"
                "FETCH_SIZE / WRITE_SIZE count L2 misses (requests that leave the XCD's L2 for the "
                "Infinity Cache / HBM), hence the l2_miss_* names; TCC_EA0_{RDREQ,WRREQ_WRITE}_DRAM_32B "
                "count the 32-byte requests of those addressed to DRAM, which still include Infinity-Cache "
                "hits (the copy calibration shows how they relate to bytes moved).\n"
                "valu_busy_pct / mfma_util_pct are derived from the raw counters with rocprofiler-sdk's "
                "formulas; sdk_* are the SDK's own derived counters from a separate pass.\n"
                "Times, rates and the effective clock (GRBM_GUI_ACTIVE cycles per ns) use the measured "
                "launches' durations from the kernel-trace pass without counters "
                "(kernel_ns_median_under_pmc is the same launches' duration in the counter pass). "
                "GRBM_GUI_ACTIVE covers a little time around each dispatch, so for short kernels "
                "(tens of us) the effective clock reads high and the MFMA utilisation low, and the raw and "
                "SDK figures, taken in different passes, can differ by more than the 10 % the "
                "*_agrees_with_sdk flags allow.\n")
        with open(os.path.join(profiles, f"counters_{w}.md"), "w") as f:
            f.write(text)
        print(f"{w}: {s['config']} {s['l2_miss_bytes_per_launch']:.4g} L2-miss B/launch")
    with open(path, "w") as f:
        json.dump(table, f, indent=2)
        f.write("\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("target")
    t.add_argument("--workload", required=True)
    t.add_argument("--iters", type=int, default=10)
    t.add_argument("--config", default=None)
    t.add_argument("--warmup", type=int, default=0)
    r = sub.add_parser("run")
    r.add_argument("--workload", required=True)
    r.add_argument("--iters", type=int, default=10)
    r.add_argument("--config", default=None)
    r.add_argument("--out", required=True)
    r.add_argument("--warmup", type=int, default=-1,
                   help="unprofiled launches before the measured ones (default: about 1.5 s of them)")
    c = sub.add_parser("collect")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    if a.mode == "target":
        _target(a)
    elif a.mode == "run":
        run(a)
    else:
        collect(a.dirs, a.profiles)


if __name__ == "__main__":
    main()
