"""Read rocprofv3 result databases (rocpd SQLite) and summarise them.

    python -m rope_frequency_pair_amd.rocprof_summary stats <run_results.db>
    python -m rope_frequency_pair_amd.rocprof_summary counters <run_results.db> [<db> ...]
    python -m rope_frequency_pair_amd.rocprof_summary traffic --fetch <db> --write <db> \
        --kernel prefill_kernel --copy-bytes 1073741824 --sha <kernel sha> --out <json>

``stats`` prints per-kernel call counts and durations (the --stats summary);
``counters`` prints the mean per-dispatch value of every collected counter
per kernel; ``traffic`` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of a
kernel into bytes, scaled by what the same counters read for the plain device
copy of ``--copy-bytes`` bytes that bench.py --copy-calibration runs first, and
writes the JSON bench.py reads for the roofline's ``traffic`` field.
"""

import argparse
import collections
import json
import sqlite3
import statistics
import sys


def _short(name, width=60):
    if name.startswith("void "):
        name = name[5:].replace("(anonymous namespace)::", "")
        name = name.split("(")[0]
    return name if len(name) <= width else name[:width - 3] + "..."


def kernel_stats(db):
    con = sqlite3.connect(db)
    rows = collections.defaultdict(list)
    for name, dur in con.execute("select name, duration from kernels"):
        rows[name].append(dur)
    out = []
    for name, d in rows.items():
        out.append({"name": name, "calls": len(d), "total_ns": sum(d), "avg_ns": statistics.mean(d),
                    "min_ns": min(d), "max_ns": max(d)})
    out.sort(key=lambda r: -r["total_ns"])
    return out


def counters(db):
    """{kernel name: {counter: [value per dispatch]}} (values summed over instances)."""
    con = sqlite3.connect(db)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for kn, did, cn, val in con.execute(
            "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
        per[(did, cn)]["v"] += val
        names[did] = kn
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (did, cn), d in per.items():
        out[names[did]][cn].append(d["v"])
    return out


def _print_stats(db):
    print(f"kernel statistics from {db}\n")
    print("| kernel | calls | avg (us) | min (us) | max (us) | total (ms) |")
    print("|---|---|---|---|---|---|")
    for r in kernel_stats(db):
        print(f"| {_short(r['name'])} | {r['calls']} | {r['avg_ns'] / 1e3:.1f} | {r['min_ns'] / 1e3:.1f} | "
              f"{r['max_ns'] / 1e3:.1f} | {r['total_ns'] / 1e6:.2f} |")


def _print_counters(dbs):
    for db in dbs:
        print(f"\ncounters from {db} (mean per dispatch)\n")
        print("| kernel | counter | dispatches | mean |")
        print("|---|---|---|---|")
        for kn, cs in counters(db).items():
            for cn, vals in sorted(cs.items()):
                print(f"| {_short(kn)} | {cn} | {len(vals)} | {statistics.mean(vals):.6g} |")


def traffic(fetch_db, write_db, kernel, copy_bytes, copy_kernel="copy"):
    def mean_for(db, counter, match):
        vals = []
        for kn, cs in counters(db).items():
            if match(kn) and counter in cs:
                vals += cs[counter]
        return statistics.mean(vals) if vals else None

    is_k = lambda kn: kernel in kn
    is_copy = lambda kn: copy_kernel in kn and kernel not in kn
    f_k, f_c = mean_for(fetch_db, "FETCH_SIZE", is_k), mean_for(fetch_db, "FETCH_SIZE", is_copy)
    w_k, w_c = mean_for(write_db, "WRITE_SIZE", is_k), mean_for(write_db, "WRITE_SIZE", is_copy)
    fetch_scale = copy_bytes / f_c if f_c else None
    write_scale = copy_bytes / w_c if w_c else None
    return {
        "fetch_kib": f_k, "write_kib": w_k, "copy_fetch_kib": f_c, "copy_write_kib": w_c,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "fetch_bytes": f_k * fetch_scale if f_k and fetch_scale else None,
        "write_bytes": w_k * write_scale if w_k and write_scale else None,
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    c = sub.add_parser("counters")
    c.add_argument("db", nargs="+")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--sha", default=None)
    t.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        _print_stats(a.db)
    elif a.cmd == "counters":
        _print_counters(a.db)
    else:
        r = traffic(a.fetch, a.write, a.kernel, a.copy_bytes, a.copy_kernel)
        r["kernel"] = a.kernel
        r["kernel_sha"] = a.sha
        r["traffic_bytes"] = (r["fetch_bytes"] or 0) + (r["write_bytes"] or 0) if r["fetch_bytes"] else None
        txt = json.dumps(r, indent=1)
        if a.out:
            with open(a.out, "w") as f:
                f.write(txt + "\n")
        print(txt)


if __name__ == "__main__":
    sys.exit(main())
