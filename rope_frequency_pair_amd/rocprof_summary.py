"""Read rocprofv3 result databases (rocpd SQLite) and summarise them.

    python -m rope_frequency_pair_amd.rocprof_summary stats <run_results.db>
    python -m rope_frequency_pair_amd.rocprof_summary counters <run_results.db> [<db> ...]
    python -m rope_frequency_pair_amd.rocprof_summary dispatches <run_results.db> \
        [--kernel SUBSTR] [--skip N] [--first N]
    python -m rope_frequency_pair_amd.rocprof_summary sequence <run_results.db> --kernel SUBSTR \
        --counter NAME [--copy-bytes N]
    python -m rope_frequency_pair_amd.rocprof_summary traffic --fetch <db> --write <db> \
        --kernel prefill_kernel --copy-bytes 1073741824 --sha <kernel sha> --out <json>

``stats`` prints per-kernel call counts and durations (the --stats summary);
``dispatches`` groups the dispatches of each kernel by launch grid, in launch
order (optionally skipping the first N of a group and keeping the next M), so
one workload's launches can be read apart from the others';
``counters`` prints the mean per-dispatch value of every collected counter
per kernel; ``sequence`` lists one counter per dispatch in dispatch order (so
launches of one kernel with different arguments can be told apart), in bytes
when the calibration copy's size is given; ``traffic`` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of a
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


def dispatch_groups(db, kernel=None, skip=0, first=None):
    con = sqlite3.connect(db)
    groups = collections.OrderedDict()
    for name, dur, gx, gy, gz, wx in con.execute(
            "select name, duration, grid_x, grid_y, grid_z, workgroup_x from kernels order by start"):
        if kernel and kernel not in name:
            continue
        groups.setdefault((name, gx, gy, gz, wx), []).append(dur)
    out = []
    for (name, gx, gy, gz, wx), d in groups.items():
        d = d[skip:]
        if first is not None:
            d = d[:first]
        if d:
            out.append({"name": name, "grid": (gx, gy, gz), "wg": wx, "calls": len(d),
                        "avg_ns": statistics.mean(d), "min_ns": min(d), "max_ns": max(d)})
    return out


def _print_dispatches(db, kernel, skip, first):
    print(f"dispatches grouped by launch grid, from {db}" + (f" (skip {skip}, first {first})" if skip or first else ""))
    print()
    print("| kernel | grid (threads) | workgroup | calls | avg (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|---|---|")
    for r in dispatch_groups(db, kernel, skip, first):
        g = "x".join(str(x) for x in r["grid"])
        print(f"| {_short(r['name'])} | {g} | {r['wg']} | {r['calls']} | {r['avg_ns'] / 1e3:.1f} | "
              f"{r['min_ns'] / 1e3:.1f} | {r['max_ns'] / 1e3:.1f} |")


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


def traffic(fetch_db, write_db, kernel, copy_bytes, copy_kernel="copyBuffer"):
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


def sequence(db, kernel, counter, copy_bytes=None, copy_kernel="copyBuffer"):
    """Every dispatch of the kernels whose name contains ``kernel``, in
    dispatch order, with its value of ``counter`` (summed over instances; the
    name ``duration`` reads a kernel-trace database's durations in ns) and,
    given the byte size of bench.py's calibration copy, that value in bytes
    scaled as the copy reads."""
    con = sqlite3.connect(db)
    per = collections.OrderedDict()
    if counter == "duration":       # a kernel-trace database: durations in ns
        for i, (kn, dur) in enumerate(con.execute("select name, duration from kernels order by start")):
            per[i] = [kn, float(dur)]
        copy_bytes = None
    else:
        for kn, did, cn, val in con.execute(
                "select kernel_name, dispatch_id, counter_name, value from counters_collection "
                "order by dispatch_id"):
            if cn != counter:
                continue
            per.setdefault(did, [kn, 0.0])
            per[did][1] += val
    scale = None
    if copy_bytes:
        copies = [v for kn, v in per.values() if copy_kernel in kn]
        scale = copy_bytes / copies[0] if copies and copies[0] else None
    out = []
    for did, (kn, v) in per.items():
        if kernel in kn:
            out.append({"dispatch": did, "name": kn, "value": v,
                        "bytes": v * scale if scale else None})
    return out, scale


def _print_sequence(db, kernel, counter, copy_bytes):
    rows, scale = sequence(db, kernel, counter, copy_bytes)
    print(f"{counter} per dispatch of kernels matching '{kernel}', in dispatch order, from {db}"
          + (f"; bytes = value x {scale:.6g} (the calibration copy)" if scale else ""))
    print()
    print(f"| dispatch | kernel | {counter} | bytes |")
    print("|---|---|---|---|")
    for r in rows:
        b = f"{r['bytes']:.6g}" if r["bytes"] is not None else "-"
        print(f"| {r['dispatch']} | {_short(r['name'])} | {r['value']:.6g} | {b} |")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    dsp = sub.add_parser("dispatches")
    dsp.add_argument("db")
    dsp.add_argument("--kernel", default=None)
    dsp.add_argument("--skip", type=int, default=0)
    dsp.add_argument("--first", type=int, default=None)
    c = sub.add_parser("counters")
    c.add_argument("db", nargs="+")
    q = sub.add_parser("sequence")
    q.add_argument("db")
    q.add_argument("--kernel", required=True)
    q.add_argument("--counter", required=True)
    q.add_argument("--copy-bytes", type=int, default=None)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-kernel", default="copyBuffer")
    t.add_argument("--sha", default=None)
    t.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        _print_stats(a.db)
    elif a.cmd == "dispatches":
        _print_dispatches(a.db, a.kernel, a.skip, a.first)
    elif a.cmd == "counters":
        _print_counters(a.db)
    elif a.cmd == "sequence":
        _print_sequence(a.db, a.kernel, a.counter, a.copy_bytes)
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
