"""Shape-keyed autotuner: times every kernel configuration that can run a
problem and writes the fastest into the tuning table the library loads
(``tune_gfx950.txt`` beside the package by default).

    python -m dense_gemm_12_amd.autotune [--out PATH] [--workload NAME ...]

Problems are the named workloads (their own seeded inputs: the data moves
the chip's clock under MFMA load, so tuning on other data would mislead) and
the tuning shapes of ``gemm_inputs`` (2048^3 to 8192^3 in every layout and
output-type class the workloads leave out).
Each configuration gets a warm-up, then ``--trials`` timed runs of enough
launches to pass ``--min-ms`` (at most 200), each launch timed on its own
with HIP events on the launch stream right after a 512 MiB buffer is
overwritten; the median launch decides.  Timing launches back to back
instead (``--warm``) ranks some tiles well above where they land inside a
program: the 4-wave 256 x 256 fp16 tile is 12-20% faster when it follows
itself than after any other kernel, while the 8-wave one does not care.  Table rows are

    <in> <c> <ta> <tb> <M> <N> <K> <config> [ws [s=<splits>]]

and the library matches a problem to the nearest row of the same type and
layout class (log-distance in M, N, K).  The table also records, per
configuration, the best fraction of the type's peak it reached here
(``rate <in> <config> <fraction>``); the library's cost model uses these to
rank configurations for shapes no rule is near, and to drop a neighbouring
shape's rule that it expects to be clearly slower.  Rows tagged ``ws`` were tuned
through gemm_ex with a workspace (split-K and operand repacking allowed) and
apply only to such calls; a workload gets one when the planner would split
or repack it, and its split count is tuned too (``s=N``; without it the
planner's fill rule decides).  The per-configuration timings are
kept as comments.
"""
from __future__ import annotations

import argparse
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)


SPLIT_CHOICES = (0, 4, 8, 16, 32)  # workspace pass: the planner's fill rule, then fixed counts
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}


FLUSH_BYTES = 512 << 20  # above the chip's last-level cache (256 MB)
MAX_COLD_REPS = 200


def time_config(mg, torch, A, B, C, w, cfg, trials, min_ms, workspace=None, splits=0, flush=None):
    """Median time of one call in ms.  With ``flush`` (a CUDA tensor of at
    least FLUSH_BYTES), every timed call runs alone between its own events
    right after the buffer is overwritten, so it starts with cold caches and
    after another kernel, as a GEMM inside a larger program does; without it,
    calls run back to back and the per-call average of each trial counts."""
    stream = torch.cuda.current_stream()
    call = lambda: mg.gemm(A, B, C, alpha=w["alpha"], beta=w["beta"], trans_a=w["ta"],
                           trans_b=w["tb"], config=cfg, stream=stream, workspace=workspace,
                           splits=splits)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    call()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    reps = max(5, int(min_ms / one) + 1)
    for _ in range(3):
        call()
    times = []
    if flush is not None:
        reps = min(reps, MAX_COLD_REPS)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for _ in range(trials):
            for a, b in ev:
                flush.zero_()
                a.record(stream)
                call()
                b.record(stream)
            torch.cuda.synchronize()
            times += [a.elapsed_time(b) for a, b in ev]
        return statistics.median(times)
    for _ in range(trials):
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    return statistics.median(times)


def _shapes():
    import gemm_inputs as gi
    return {**gi.WORKLOADS, **gi.TUNING_SHAPES}


def _prefer_consistent(lines, picks, log, margin=0.02):
    """Near-ties: when the runner-up is within `margin` of the winner and is
    what the nearest tuned shapes of the same type and layout chose, take the
    runner-up, so that one shape class does not flip between configurations
    on run-to-run noise.  Only peers whose own pick was decisive (their
    runner-up more than `margin` behind) count, and every peer at the nearest
    distance must agree, so one noisy pick cannot pull its neighbours along."""
    import math
    shapes = _shapes()
    chosen = {(n, t): r[0][1] for n, t, r in picks}
    decisive = {(n, t) for n, t, r in picks if len(r) < 2 or r[1][0] > r[0][0] * (1 + margin)}
    for n, t, ranked in picks:
        if (n, t) in decisive:
            continue
        w = shapes[n]
        key = (w["in_dtype"], w["c_dtype"], w["ta"], w["tb"])
        dist = lambda o: sum(abs(math.log2((shapes[o][d] + 1) / (w[d] + 1))) for d in "MNK")
        peers = [o for o, ot in chosen if ot == t and o != n and (o, ot) in decisive and
                 (shapes[o]["in_dtype"], shapes[o]["c_dtype"], shapes[o]["ta"], shapes[o]["tb"]) == key]
        if not peers:
            continue
        d0 = min(dist(o) for o in peers)
        nearest = [o for o in peers if dist(o) == d0]
        if {chosen[(o, t)] for o in nearest} == {ranked[1][1]} and ranked[1][2] == ranked[0][2]:
            old, new = ranked[0][1], ranked[1][1]
            log(f"{n}{t}: {old} and {new} within {margin:.0%}; taking {new} as {', '.join(nearest)} do")
            lines = [l.replace(f" {old}", f" {new}", 1) if (not l.startswith("#") and l.split()[4:7] ==
                     [str(w["M"]), str(w["N"]), str(w["K"])] and ((" ws" in l) == (t == " ws"))) else l
                     for l in lines]
    return lines


def tune(names, out, trials=3, min_ms=20.0, log=print, cold=True):
    import torch
    import dense_gemm_12_amd as mg
    import gemm_inputs as gi
    os.environ["MGEMM_NO_TUNE_TABLE"] = "1"  # time configurations, not an older table's picks
    mg.load()
    dev = torch.device("cuda:0")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev) if cold else None
    picks = []  # (name, tag, ranked [(ms, config, splits)]) in tuning order
    rates = {}  # (input type, config) -> best fraction of peak over the plain calls
    lines = ["# dense_gemm_12_amd tuning table for gfx950 (MI355X); written by autotune.py",
             "# <in> <c> <ta> <tb> <M> <N> <K> <config> [ws [s=N]]; comments: the three fastest candidates"]
    shapes = _shapes()
    for name in names:
        w = shapes[name]
        A, B, C = gi.workload_inputs(name)
        Ad, Bd = A.to(dev), B.to(dev)
        Cd = (C.to(dev) if C is not None else
              torch.zeros((w["M"], w["N"]), dtype=gi.DTYPES[w["c_dtype"]], device=dev))
        codes = mg.DTYPE_CODES
        wsb = mg.workspace_size(codes[w["in_dtype"]], codes[w["c_dtype"]], int(w["ta"]), int(w["tb"]),
                                w["M"], w["N"], w["K"], Ad.stride(0), Bd.stride(0))
        # plain calls, then (when gemm_ex would split or repack) calls with a
        # workspace, each tuned into its own rule
        passes = [("", None, (0,))]
        if wsb:
            # room for the operand copies and the largest split count tried
            big = wsb + max(SPLIT_CHOICES) * w["M"] * w["N"] * 4
            passes.append((" ws", torch.empty(big, dtype=torch.uint8, device=dev), SPLIT_CHOICES))
        for tag, ws, split_choices in passes:
            results = []
            for cfg in range(mg.num_configs(w["in_dtype"])):
                cname = mg.config_name(w["in_dtype"], cfg)
                for sp in split_choices:
                    try:
                        ms = time_config(mg, torch, Ad, Bd, Cd, w, cfg, trials, min_ms, workspace=ws,
                                         splits=sp, flush=flush)
                    except mg.MgemmError as e:
                        if e.status != mg.MG_EUNSUPPORTED:
                            raise
                        break
                    flops = 2.0 * w["M"] * w["N"] * w["K"]
                    if not tag:
                        frac = flops / ms / 1e9 / PEAK_TFLOPS[w["in_dtype"]]
                        rates[(w["in_dtype"], cname)] = max(frac, rates.get((w["in_dtype"], cname), 0.0))
                    label = cname + (f" s={sp}" if sp else "")
                    results.append((ms, cname, sp))
                    log(f"{name + tag:28s} {label:38s} {ms * 1e3:10.1f} us {flops / ms / 1e9:9.1f} TFLOPS")
            if not results:
                continue
            results.sort()
            tie_note = ""
            if flush is not None and len(results) > 1:
                # Near-ties of the cold time (within 1 %) go to the faster
                # back-to-back (warm) call: at this margin cold timings differ
                # by run-to-run noise, while warm ones can still tell the
                # kernels apart.
                near = [r for r in results[:3] if r[0] <= results[0][0] * 1.01]
                if len(near) > 1:
                    warm = [(time_config(mg, torch, Ad, Bd, Cd, w, mg.config_id(w["in_dtype"], c), trials, min_ms,
                                         workspace=ws, splits=sp), (ms, c, sp)) for ms, c, sp in near]
                    best_warm, best_r = min(warm)
                    if best_r != results[0]:
                        log(f"{name + tag}: cold times within 1 %; {best_r[1]} is fastest warm "
                            f"({best_warm * 1e3:.1f} us)")
                        results.remove(best_r)
                        results.insert(0, best_r)
                        tie_note = f" (near-tie: {best_r[1]} fastest warm, {best_warm * 1e3:.1f}us)"
            picks.append((name, tag, results))
            best_ms, best, best_sp = results[0]
            if best_sp:
                # a fixed split count must beat the fill rule by more than noise
                auto = [ms for ms, c, sp in results if c == best and sp == 0]
                if auto and auto[0] <= best_ms * 1.02:
                    best_sp = 0
            rule_tag = tag + (f" s={best_sp}" if best_sp else "")
            lines.append(f"# {name}{tag}: " + ", ".join(
                f"{c}{'/s=%d' % sp if sp else ''}={ms * 1e3:.1f}us" for ms, c, sp in results[:3]) + tie_note)
            lines.append(f"{w['in_dtype']} {w['c_dtype']} {'T' if w['ta'] else 'N'} {'T' if w['tb'] else 'N'} "
                         f"{w['M']} {w['N']} {w['K']} {best}{rule_tag}")
        del Ad, Bd, Cd
        torch.cuda.empty_cache()
    lines = _prefer_consistent(lines, picks, log)
    # the planner's cost model ranks configurations on shapes no rule is near
    # by these measured rates
    lines.append("# rate <in> <config> <best fraction of the type's peak over the plain calls above> "
                 "<workgroups per CU>")
    for (t, c), f in sorted(rates.items()):
        occ = mg.config_occupancy(t, mg.config_id(t, c))
        if f > 0 and occ > 0:
            lines.append(f"rate {t} {c} {min(f, 1.0):.4f} {occ}")
    tmp = out + ".tmp"
    with open(tmp, "w") as f:
        f.write("\n".join(lines) + "\n")
    os.replace(tmp, out)
    log(f"wrote {out}")
    return out


def main():
    import gemm_inputs as gi
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "tune_gfx950.txt"))
    ap.add_argument("--workload", nargs="*", default=list(gi.WORKLOADS) + list(gi.TUNING_SHAPES))
    ap.add_argument("--trials", type=int, default=3)
    ap.add_argument("--min-ms", type=float, default=20.0)
    ap.add_argument("--warm", action="store_true",
                    help="time calls back to back instead of each after a cache scrub")
    a = ap.parse_args()
    t0 = time.time()
    tune(a.workload, a.out, a.trials, a.min_ms, log=lambda s: print(s, flush=True), cold=not a.warm)
    print(f"tuning took {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main()
