#!/usr/bin/env python3
"""Short text / JSON summaries of rocprofv3 result databases, for the profiles/ folder.

rocprofv3 (ROCm 7.x) writes one SQLite database per run (``<name>_results.db``).  This
script reads its ``kernels`` view (kernel trace) or ``counters_collection`` view (--pmc runs)
and writes the few figures the benchmark and the design notes use:

    python profile_summary.py trace RUN.db [RUN.db ...] --out profiles/NAME.txt --command "..."
        per-kernel calls, average / min / max duration, share of GPU time, registers and LDS.

    python profile_summary.py traffic --fetch F.db --write W.db --kernel REGEX --calib-mib MIB
        --source SRC --workload NAME --out profiles/traffic_NAME.json
        --fetch-command "..." --write-command "..."
        HBM bytes per launch of the kernels matching REGEX: FETCH_SIZE and WRITE_SIZE (KiB per
        dispatch), each scaled by the reading of the same counter for a plain streaming kernel
        of known size (torch.neg over MIB MiB of fp32: MIB MiB read and MIB MiB written).  The
        source file's sha256 is stored so that the benchmark only reports the figure while the
        kernel source is unchanged.

    python profile_summary.py counters RUN.db [RUN.db ...] --kernel REGEX --out profiles/NAME.txt
        --command "..." [--command "..."]
        every counter the runs collected for the kernels matching REGEX, averaged per dispatch
        (each counter summed over the rows of a dispatch), with the dispatches' average duration.

    python profile_summary.py mfma RUN.db --kernel REGEX --workload NAME --out profiles/mfma_NAME.json
        --command "..."
        counter-based MFMA-pipe utilisation of the kernels matching REGEX: SQ_VALU_MFMA_BUSY_CYCLES
        (the MFMA unit's busy cycles summed over every SIMD) over 1024 SIMDs x the dispatch's
        duration x the nominal 2.4 GHz clock.

Records (traffic, mfma) store the library hash of ``curvature_conditioned_query_amd.build``
(every source, header and compile flag), so the benchmark only reports a figure while the built
code is the one it was measured on.
"""

from __future__ import annotations

import argparse
import collections
import json
import re
import sqlite3
import sys

CALIB_KERNEL = r"neg_kernel"
SIMDS = 1024            # MI355X: 256 compute units x 4 SIMDs
NOMINAL_CLOCK_HZ = 2.4e9


def library_sha256() -> str:
    from curvature_conditioned_query_amd.build import library_sha256 as _sha
    return _sha()


def _short(name: str) -> str:
    name = name.replace("void ", "")
    return name.split("(")[0][:96]


def trace_rows(db_path):
    db = sqlite3.connect(db_path)
    cur = db.cursor()
    return cur.execute("select name, duration, grid_x, grid_y, workgroup_x, vgpr_count, accum_vgpr_count, "
                       "lds_size from kernels").fetchall()


def trace_summary(paths, command, title):
    out = [f"# {title}", f"# command: {command}", ""]
    for path in paths:
        rows = trace_rows(path)
        agg = collections.OrderedDict()
        for name, dur, gx, gy, wx, v, a, lds in rows:
            key = (_short(name), gx, gy, wx)
            e = agg.setdefault(key, dict(n=0, tot=0, mn=float("inf"), mx=0, v=v, a=a, lds=lds))
            e["n"] += 1
            e["tot"] += dur
            e["mn"] = min(e["mn"], dur)
            e["mx"] = max(e["mx"], dur)
        tot = sum(e["tot"] for e in agg.values()) or 1
        out.append(f"## {path.split('/')[-1]}")
        out.append(f"{'kernel':<96} {'grid(threads)':>14} {'wg':>4} {'calls':>5} {'avg_us':>9} {'min_us':>9} "
                   f"{'max_us':>9} {'time%':>6} {'vgpr':>5} {'lds_B':>7}")
        for (k, gx, gy, wx), e in sorted(agg.items(), key=lambda kv: -kv[1]["tot"]):
            out.append(f"{k:<96} {f'{gx}x{gy}':>14} {wx:>4} {e['n']:>5} {e['tot'] / e['n'] / 1e3:>9.2f} "
                       f"{e['mn'] / 1e3:>9.2f} {e['mx'] / 1e3:>9.2f} {100 * e['tot'] / tot:>6.1f} "
                       f"{e['v']:>5} {e['lds']:>7}")
        out.append("")
    return "\n".join(out)


def counter_per_dispatch(db_path, counter, kernel_regex, largest_only=False):
    """Average per-dispatch value of `counter` over the dispatches whose kernel name matches
    (with largest_only, over those within 5 % of the largest: the calibration copies, not the
    small launches of the same torch kernel that building the inputs may make)."""
    db = sqlite3.connect(db_path)
    cur = db.cursor()
    rows = cur.execute("select kernel_name, dispatch_id, counter_name, value, duration from counters_collection").fetchall()
    pat = re.compile(kernel_regex)
    per = collections.defaultdict(float)
    dur = {}
    names = set()
    for k, d, c, v, du in rows:
        if c != counter or not pat.search(k):
            continue
        per[d] += v
        dur[d] = du
        names.add(_short(k))
    if not per:
        raise SystemExit(f"{db_path}: no {counter} rows for kernels matching {kernel_regex!r}")
    if largest_only:
        top = max(per.values())
        per = {d: v for d, v in per.items() if v >= 0.95 * top}
        dur = {d: dur[d] for d in per}
    n = len(per)
    return sum(per.values()) / n, n, sum(dur.values()) / n / 1e3, sorted(names)


def traffic_summary(a):
    f_k, n_f, us_f, names = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    w_k, n_w, us_w, _ = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cf_k, _, _, _ = counter_per_dispatch(a.fetch, "FETCH_SIZE", CALIB_KERNEL, largest_only=True)
    cw_k, _, _, _ = counter_per_dispatch(a.write, "WRITE_SIZE", CALIB_KERNEL, largest_only=True)
    calib_bytes = a.calib_mib * (1 << 20)
    s_fetch = calib_bytes / (cf_k * 1024.0)
    s_write = calib_bytes / (cw_k * 1024.0)
    fetch_b = f_k * 1024.0 * s_fetch
    write_b = w_k * 1024.0 * s_write
    return {
        "workload": a.workload,
        "kernel": names,
        "source": a.source,
        "library_sha256": library_sha256(),
        "dispatches": {"fetch_run": n_f, "write_run": n_w},
        "avg_duration_us_under_counters": {"fetch_run": round(us_f, 2), "write_run": round(us_w, 2)},
        "fetch_kib_per_dispatch": round(f_k, 1),
        "write_kib_per_dispatch": round(w_k, 1),
        "calibration": {"kernel": "torch.neg on fp32", "bytes_read": calib_bytes, "bytes_written": calib_bytes,
                        "fetch_kib": round(cf_k, 1), "write_kib": round(cw_k, 1),
                        "fetch_scale": round(s_fetch, 4), "write_scale": round(s_write, 4)},
        "hbm_read_bytes_per_launch": round(fetch_b),
        "hbm_write_bytes_per_launch": round(write_b),
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "commands": {"fetch": a.fetch_command, "write": a.write_command},
    }


def mfma_summary(a):
    busy, n, us, names = counter_per_dispatch(a.db, "SQ_VALU_MFMA_BUSY_CYCLES", a.kernel)
    frac = busy / (SIMDS * us * 1e-6 * NOMINAL_CLOCK_HZ)
    return {
        "workload": a.workload,
        "kernel": names,
        "library_sha256": library_sha256(),
        "dispatches": n,
        "avg_duration_us_under_counters": round(us, 2),
        "mfma_busy_cycles_per_dispatch": round(busy, 1),
        "mfma_busy_frac": round(frac, 4),
        "definition": "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x avg dispatch duration x 2.4 GHz)",
        "command": a.command,
    }


def counters_summary(paths, kernel_regex, commands, title):
    pat = re.compile(kernel_regex)
    out = [f"# {title}", f"# kernels matching: {kernel_regex}"]
    out += [f"# command: {c}" for c in commands]
    out.append("")
    out.append(f"{'counter':<32} {'per dispatch':>16} {'dispatches':>10} {'avg_us':>9}  run")
    for path in paths:
        db = sqlite3.connect(path)
        rows = db.cursor().execute(
            "select kernel_name, dispatch_id, counter_name, value, duration from counters_collection").fetchall()
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        dur = collections.defaultdict(dict)
        for k, d, c, v, du in rows:
            if pat.search(k):
                per[c][d] += v
                dur[c][d] = du
        for c in sorted(per):
            vals = per[c]
            n = len(vals)
            us = sum(dur[c].values()) / n / 1e3
            out.append(f"{c:<32} {sum(vals.values()) / n:>16.5g} {n:>10} {us:>9.2f}  {path.split('/')[-1]}")
    out.append("")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dbs", nargs="+")
    t.add_argument("--out", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="rocprofv3 --kernel-trace --stats")
    q = sub.add_parser("counters")
    q.add_argument("dbs", nargs="+")
    q.add_argument("--kernel", required=True)
    q.add_argument("--out", required=True)
    q.add_argument("--command", action="append", required=True)
    q.add_argument("--title", default="rocprofv3 --pmc counters")
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--calib-mib", type=int, required=True)
    c.add_argument("--source", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--fetch-command", required=True)
    c.add_argument("--write-command", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("db")
    m.add_argument("--kernel", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.mode == "mfma":
        rec = mfma_summary(a)
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print(json.dumps(rec, indent=1))
    elif a.mode == "trace":
        text = trace_summary(a.dbs, a.command, a.title)
        with open(a.out, "w") as fh:
            fh.write(text + "\n")
        print(text)
    elif a.mode == "counters":
        text = counters_summary(a.dbs, a.kernel, a.command, a.title)
        with open(a.out, "w") as fh:
            fh.write(text + "\n")
        print(text)
    else:
        rec = traffic_summary(a)
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print(json.dumps(rec, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
