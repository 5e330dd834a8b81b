#!/usr/bin/env python3
"""Turn rocprofv3 output of bench.py runs into the summaries kept under profiles/.

Reads the rocpd SQLite databases of five runs of one workload (all from the repository root):

    rocprofv3 --kernel-trace --stats -T -d T -o trace -- python3 bench.py --workload W --only --steps 100 --warmup 10 --no-cpu-baseline
    rocprofv3 --pmc FETCH_SIZE -T -d F -o fetch -- python3 bench.py --workload W --only --steps 3 --warmup 1 --no-cpu-baseline --eager
    rocprofv3 --pmc WRITE_SIZE -T -d R -o write -- python3 bench.py --workload W --only --steps 3 --warmup 1 --no-cpu-baseline --eager
    rocprofv3 --pmc FETCH_SIZE -T -d CF -o cf -- python3 bench.py --copy-calibration 1024
    rocprofv3 --pmc WRITE_SIZE -T -d CW -o cw -- python3 bench.py --copy-calibration 1024

and writes profiles/decode_<W>.md plus the workload's entry of profiles/decode_counters.json
(the HBM bytes per decode call that bench.py reports as roofline.traffic, keyed by a hash of
the decode kernel's code so that a changed kernel reports null until it is profiled again).

    python profile_report.py W T F R CF CW
    python profile_report.py --kernels prefill_kernel --name prefill_70b --cmd "--op prefill" \
        [--timed K] [--counters-key KEY] T F R CF CW

The second form summarises other kernels of other bench modes into profiles/<name>.md (the trace
and counter runs then use `bench.py <cmd>` in place of `--workload W`).  With --timed K the
summary also gives the first kernel's statistics over its last K dispatches (the bench's timed
calls, after the warm-up).  With --counters-key the HBM bytes per launch of the first kernel go
into profiles/prefill_counters.json under that key, with the hash of the prefill kernel's code.
"""
from __future__ import annotations

import glob
import json
import os
import sqlite3
import sys

from bench import COUNTERS, KERNEL_SOURCE, PREFILL_COUNTERS, PREFILL_SOURCE, ROOT, source_hash
DECODE_KERNELS = ("decode_piece_kernel",)  # cut segments are merged inside it
COPY_BYTES = 1 << 30

TRACE_STEPS = 100  # timed steps of the traced decode run: its last TRACE_STEPS dispatches
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -T -d <out> -o trace -- python3 bench.py --workload {w} --only "
             f"--steps {TRACE_STEPS} --warmup 10 --no-cpu-baseline")
PMC_CMD = ("timeout -s KILL 150 rocprofv3 --pmc {c} -T -d <out> -o {o} -- python3 bench.py --workload {w} --only "
           "--steps 3 --warmup 1 --no-cpu-baseline --eager")
COPY_CMD = "timeout -s KILL 90 rocprofv3 --pmc {c} -T -d <out> -o {o} -- python3 bench.py --copy-calibration 1024"


def _db(d):
    hits = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    if not hits:
        raise SystemExit(f"no rocpd database under {d}")
    return sqlite3.connect(hits[0])


def _short(name):
    return name.split("(")[0].split("<")[0].split("::")[-1].strip()


def trace_stats(d):
    con = _db(d)
    rows = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    launch = {}
    for r in con.execute("select name, grid_x, workgroup_x, vgpr_count, accum_vgpr_count, sgpr_count, lds_size, "
                         "scratch_size from kernels"):
        launch.setdefault(_short(r[0]), r[1:])
    return [(_short(n), c, t, a, p) for n, c, t, a, p in rows], launch  # durations in us


def counter_kib(d, counter):
    """Average value of `counter` per dispatch, per kernel (KiB for FETCH_SIZE / WRITE_SIZE)."""
    con = _db(d)
    out = {}
    for name, v, n in con.execute("select kernel_name, avg(value), count(*) from counters_collection "
                                  "where counter_name = ? group by kernel_name", (counter,)):
        out[_short(name)] = (v, n)
    return out


def main(argv):
    kernels, name, cmd, timed, ckey = DECODE_KERNELS, None, None, 0, None
    while argv and argv[0].startswith("--"):
        opt, val, argv = argv[0], argv[1], argv[2:]
        if opt == "--kernels":
            kernels = tuple(val.split(","))
        elif opt == "--name":
            name = val
        elif opt == "--cmd":
            cmd = val
        elif opt == "--timed":
            timed = int(val)
        elif opt == "--counters-key":
            ckey = val
        else:
            raise SystemExit(__doc__)
    if name is None and len(argv) == 6:
        report_decode(*argv, kernels)
    elif name is not None and cmd is not None and len(argv) == 5:
        report_other(name, cmd, kernels, *argv, timed=timed, ckey=ckey)
    else:
        raise SystemExit(__doc__)


def dispatch_durations(d, kernel):
    """Durations (us) of every dispatch of `kernel`, in launch order."""
    con = _db(d)
    return [dur / 1e3 for name, dur in con.execute("select name, duration from kernels order by start")
            if _short(name) == kernel]


def dispatch_spans(d, kernel):
    """(start, end) in ns of every dispatch of `kernel`, in launch order."""
    con = _db(d)
    return [(st, en) for name, st, en in con.execute("select name, start, end from kernels order by start")
            if _short(name) == kernel]


def timed_region_lines(d, kernel, k):
    """Statistics of the last k dispatches of `kernel` (a bench run's timed steps, replayed back to back
    from multi-step graphs): durations, the gaps between consecutive ones, and the span per dispatch."""
    sp = dispatch_spans(d, kernel)[-k:]
    if len(sp) < 2:
        return [], None
    dur = sorted((en - st) / 1e3 for st, en in sp)
    gaps = sorted((sp[i + 1][0] - sp[i][1]) / 1e3 for i in range(len(sp) - 1))
    avg = sum(dur) / len(dur)
    per = (sp[-1][1] - sp[0][0]) / 1e3 / len(sp)
    return [f"Timed region ({kernel}, the last {len(sp)} dispatches: the bench's timed steps, replayed from "
            f"multi-step graphs): duration average {avg:.2f} us, median {dur[len(dur) // 2]:.2f}, min {dur[0]:.2f}, "
            f"max {dur[-1]:.2f}; gap from one dispatch's end to the next one's start median {gaps[len(gaps) // 2]:.2f} "
            f"us, min {gaps[0]:.2f}, max {gaps[-1]:.2f}; span of the region per dispatch {per:.2f} us."], per


def _calibration(cf_dir, cw_dir):
    cf, cw = counter_kib(cf_dir, "FETCH_SIZE")["copy_kernel"][0], counter_kib(cw_dir, "WRITE_SIZE")["copy_kernel"][0]
    return cf, cw, COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)


def _trace_lines(stats, launch, kernels, trace_cmd):
    L = ["Kernel trace (rocprofv3 --kernel-trace --stats), one GPU.", "", "Command (from the repository root):", "",
         "    " + trace_cmd, "", "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for n, c, t, a, p in stats:
        L.append(f"| {n} | {c} | {t:.1f} | {a:.2f} | {p:.1f} |")
    L.append("")
    for k in kernels:
        if k in launch:
            g, wg, v, ag, sg, lds, scr = launch[k]
            L.append(f"{k} launch: grid {g} threads in workgroups of {wg}; VGPR field {v}, AGPR {ag}, "
                     f"SGPR {sg}, LDS {lds} B, scratch {scr} B.")
    return L


def report_other(name, cmd, kernels, t_dir, f_dir, r_dir, cf_dir, cw_dir, timed=0, ckey=None):
    """F and R may be '-' for a trace-only summary."""
    stats, launch = trace_stats(t_dir)
    steps = f"--steps {timed} --warmup 20" if timed else "--steps 20 --warmup 5"
    trace_cmd = f"rocprofv3 --kernel-trace --stats -T -d <out> -o trace -- python3 bench.py {cmd} {steps}"
    L = [f"# {name} on MI355X (`bench.py {cmd}`)", ""] + _trace_lines(stats, launch, kernels, trace_cmd)
    timed_avg = None
    if timed:
        durs = dispatch_durations(t_dir, kernels[0])
        last = sorted(durs[-timed:])
        timed_avg = sum(last) / len(last)
        L += ["", f"{kernels[0]}: {len(durs)} dispatches in the trace; the last {len(last)} are the bench's timed "
              f"calls: average {timed_avg:.2f} us, median {last[len(last) // 2]:.2f} us, min {last[0]:.2f} us, "
              f"max {last[-1]:.2f} us (the first {len(durs) - len(last)}, warm-up and setup, average "
              f"{(sum(durs) - sum(durs[-timed:])) / max(1, len(durs) - len(last)):.2f} us)."]
    if f_dir == "-" or r_dir == "-":
        with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
            f.write("\n".join(L + [""]))
        print(name, {k: round(a, 2) for k, _, _, a, _ in stats if k in kernels})
        return
    fetch, write = counter_kib(f_dir, "FETCH_SIZE"), counter_kib(r_dir, "WRITE_SIZE")
    cf, cw, ff, wf = _calibration(cf_dir, cw_dir)
    pmc = f"timeout -s KILL 150 rocprofv3 --pmc {{c}} -T -d <out> -o {{o}} -- python3 bench.py {cmd} --steps 20 --warmup 2"
    L += ["", "## HBM traffic (rocprofv3 --pmc, one counter per run)", "", "Commands:", "",
          "    " + pmc.format(c="FETCH_SIZE", o="fetch"), "    " + pmc.format(c="WRITE_SIZE", o="write"),
          "    " + COPY_CMD.format(c="FETCH_SIZE", o="cf"), "    " + COPY_CMD.format(c="WRITE_SIZE", o="cw"), "",
          f"Calibration: bytes = FETCH_SIZE x {ff:.4f} x 1024 and WRITE_SIZE x {wf:.4f} x 1024 (copy kernel over 1 GiB).",
          "", "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | dispatches | fetched MB | written MB |",
          "|---|---|---|---|---|---|"]
    for k in kernels:
        if k in fetch and k in write:
            L.append(f"| {k} | {fetch[k][0]:.1f} | {write[k][0]:.1f} | {fetch[k][1]} | "
                     f"{fetch[k][0] * 1024 * ff / 1e6:.2f} | {write[k][0] * 1024 * wf / 1e6:.2f} |")
    L.append("")
    k0 = kernels[0]
    if ckey and k0 in fetch and k0 in write:
        sha = source_hash(PREFILL_SOURCE)
        fb, wb = fetch[k0][0] * 1024 * ff, write[k0][0] * 1024 * wf
        try:
            rec = json.load(open(PREFILL_COUNTERS))
        except (OSError, ValueError):
            rec = {}
        rec[ckey] = {"code_sha256_16": sha, "fetch_factor": ff, "write_factor": wf, "fetch_bytes": round(fb),
                     "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb),
                     "avg_us_timed_calls": None if timed_avg is None else round(timed_avg, 3)}
        with open(PREFILL_COUNTERS, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
            f.write("\n")
        L += [f"Per launch: {(fb + wb) / 1e6:.2f} MB moved beyond L2 (kernel code sha256[:16], comments and "
              f"whitespace removed: {sha}); bench.py reports it as roofline.traffic under `{ckey}`.", ""]
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(L))
    print(name, {k: round(a, 2) for k, _, _, a, _ in stats if k in kernels}, "timed avg", timed_avg)


def report_decode(w, t_dir, f_dir, r_dir, cf_dir, cw_dir, kernels=DECODE_KERNELS):
    stats, launch = trace_stats(t_dir)
    fetch, write = counter_kib(f_dir, "FETCH_SIZE"), counter_kib(r_dir, "WRITE_SIZE")
    cf, cw = counter_kib(cf_dir, "FETCH_SIZE")["copy_kernel"][0], counter_kib(cw_dir, "WRITE_SIZE")["copy_kernel"][0]
    ff, wf = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    sha = source_hash(KERNEL_SOURCE)
    avg = {n: a for n, _, _, a, _ in stats}

    entry = {"code_sha256_16": sha, "fetch_factor": ff, "write_factor": wf}
    total = 0.0
    present = [k for k in DECODE_KERNELS if k in fetch and k in write and k in avg]
    absent = [k for k in DECODE_KERNELS if k not in present]
    for k in present:
        fb = fetch[k][0] * 1024 * ff
        wb = write[k][0] * 1024 * wf
        entry[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "avg_us_trace": round(avg[k], 3)}
        total += fb + wb
    entry["hbm_bytes_per_launch"] = round(total)
    try:
        rec = json.load(open(COUNTERS))
    except (OSError, ValueError):
        rec = {}
    rec[w] = entry
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")

    region, per = timed_region_lines(t_dir, DECODE_KERNELS[0], TRACE_STEPS)
    if per is not None and DECODE_KERNELS[0] in entry:
        entry[DECODE_KERNELS[0]]["us_per_timed_step_trace"] = round(per, 3)
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    L = [f"# paged decode on MI355X: workload `{w}`", "",
         f"Kernel trace (rocprofv3 --kernel-trace --stats), one GPU: {TRACE_STEPS} timed steps twice (one graph",
         "launch per step, then the timed region proper: multi-step graph launches), 10 warm-up steps, the eager",
         "per-call timing pass, and the bench's setup (prefill appends, a 4 GiB read-ceiling probe).", "",
         "Command (from the repository root):", "", "    " + TRACE_CMD.format(w=w), "",
         "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for n, c, t, a, p in stats:
        L.append(f"| {n} | {c} | {t:.1f} | {a:.2f} | {p:.1f} |")
    L.append("")
    for k in DECODE_KERNELS:
        if k in launch:
            g, wg, v, ag, sg, lds, scr = launch[k]
            L.append(f"{k} launch: grid {g} threads in workgroups of {wg}; VGPR field {v}, AGPR {ag}, "
                     f"SGPR {sg}, LDS {lds} B, scratch {scr} B.")
    L += [""] + region
    L += ["", "With bf16 pools the step's append runs inside decode_piece_kernel (pkv_decode_step), so every",
          "kv_append call is the setup's prefill; with E4M3 pools the step's kv_append calls are the short ones.", "",
          "## HBM traffic (rocprofv3 --pmc, one counter per run)", "", "Commands:", "",
          "    " + PMC_CMD.format(c="FETCH_SIZE", o="fetch", w=w), "    " + PMC_CMD.format(c="WRITE_SIZE", o="write", w=w),
          "    " + COPY_CMD.format(c="FETCH_SIZE", o="cf"), "    " + COPY_CMD.format(c="WRITE_SIZE", o="cw"), "",
          f"Calibration: the library's copy kernel over 1 GiB reads FETCH_SIZE = {cf:.1f} KiB and WRITE_SIZE = "
          f"{cw:.1f} KiB per dispatch, so bytes = FETCH_SIZE x {ff:.4f} x 1024 and WRITE_SIZE x {wf:.4f} x 1024.", "",
          "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | dispatches | fetched MB | written MB |",
          "|---|---|---|---|---|---|"]
    for k in present:
        L.append(f"| {k} | {fetch[k][0]:.1f} | {write[k][0]:.1f} | {fetch[k][1]} | "
                 f"{entry[k]['fetch_bytes'] / 1e6:.2f} | {entry[k]['write_bytes'] / 1e6:.2f} |")
    for k in absent:
        L.append(f"| {k} | not launched | | 0 | 0 | 0 |")
    L += ["", f"Decode call total: {total / 1e6:.2f} MB moved beyond L2 per launch "
          f"(kernel code sha256[:16], comments and whitespace removed: {sha}).", ""]
    with open(os.path.join(ROOT, "profiles", f"decode_{w}.md"), "w") as f:
        f.write("\n".join(L))
    print(f"{w}: {total / 1e6:.2f} MB per decode call; " +
          ", ".join(f"{k} {avg[k]:.2f} us" for k in present) + "".join(f", {k} not launched" for k in absent))


if __name__ == "__main__":
    main(sys.argv[1:])
