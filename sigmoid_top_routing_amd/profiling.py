"""Summaries of rocprofv3 databases (the rocpd SQLite files it writes).

    python -m sigmoid_top_routing_amd.profiling kernels  DB
    python -m sigmoid_top_routing_amd.profiling counters DB
    python -m sigmoid_top_routing_amd.profiling traffic  FETCH_DB WRITE_DB \
        --kernel PATTERN --workload NAME --copy-bytes N [--source FILE ...] [--out JSON]

`kernels` prints the per-kernel call count, total and average duration of a
`--kernel-trace --stats` run. `counters` prints per-kernel averages of every
counter of a `--pmc` run. `traffic` turns two `--pmc` runs (FETCH_SIZE, then
WRITE_SIZE, KiB per dispatch) into HBM bytes per launch of one kernel: each
counter is divided by what the same counter reads, per byte, for the largest
plain device-to-device copy in the same run (a copy of --copy-bytes bytes
reads and writes exactly that many bytes), and the result is stored under
"<kernel tag>@<workload>" in profiles/traffic.json together with a digest of
the code of the kernel sources it was taken on (comments and spacing are not
part of the digest).
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import re
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def short_name(name: str) -> str:
    name = name.replace("moe::(anonymous namespace)::", "")
    return re.sub(r"\(.*\)$", "", name)[:90]


def code_text(source: str) -> str:
    """The source without comments and with whitespace collapsed: what the
    compiler sees, so a comment edit keeps a record valid."""
    source = re.sub(r"/\*.*?\*/", " ", source, flags=re.S)
    source = re.sub(r"//[^\n]*", " ", source)
    return " ".join(source.split())


def source_digest(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(HERE, "csrc", n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_table(db: str) -> str:
    cur = sqlite3.connect(db).cursor()
    rows = list(cur.execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels"))
    out = ["| kernel | calls | total us | avg us | % |", "|---|---|---|---|---|"]
    for name, calls, tot, avg, pct in rows:
        out.append(f"| `{short_name(name)}` | {calls} | {tot:.1f} | {avg:.2f} | "
                   f"{pct:.1f} |")
    return "\n".join(out)


def counter_averages(db: str):
    """{kernel: {"dispatches": n, "avg_us": t, counter: mean per dispatch}}"""
    cur = sqlite3.connect(db).cursor()
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(dict)
    for name, did, dur, cname, val in cur.execute(
            "select name, dispatch_id, duration, counter_name, counter_value from pmc_events"):
        k = short_name(name)
        acc[k][cname] += val
        disp[k][did] = dur
    res = {}
    for k, cs in acc.items():
        n = len(disp[k])
        res[k] = {"dispatches": n, "avg_us": sum(disp[k].values()) / n / 1e3,
                  **{c: v / n for c, v in cs.items()}}
    return res


def per_dispatch(db: str, counter: str):
    """[(kernel, dispatch_id, value)] for one counter."""
    cur = sqlite3.connect(db).cursor()
    vals = collections.defaultdict(float)
    names = {}
    for name, did, cname, val in cur.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if cname == counter:
            vals[did] += val
            names[did] = short_name(name)
    return [(names[d], d, v) for d, v in vals.items()]


def traffic(fetch_db, write_db, kernel, copy_bytes, copy_kernel=COPY_KERNEL):
    """HBM bytes per launch of `kernel` (a substring of its name), scaled by
    the largest plain copy (copy_kernel, a substring of its name) of
    copy_bytes bytes."""
    res = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = per_dispatch(db, counter)
        copies = [v for n, _, v in rows if copy_kernel in n]
        if not copies:
            raise SystemExit(f"{db}: no {copy_kernel} dispatch to scale {counter} by")
        factor = max(copies) * 1024.0 / copy_bytes       # counter bytes per real byte
        mine = [v for n, _, v in rows if kernel in n]
        if not mine:
            raise SystemExit(f"{db}: no dispatch of a kernel matching {kernel!r}")
        res[counter] = {"kib_per_dispatch": sum(mine) / len(mine), "dispatches": len(mine),
                        "copy_factor": factor,
                        "bytes_per_launch": sum(mine) / len(mine) * 1024.0 / factor}
    res["bytes_per_launch"] = res["FETCH_SIZE"]["bytes_per_launch"] + \
        res["WRITE_SIZE"]["bytes_per_launch"]
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("kernels")
    a.add_argument("db")
    a = sub.add_parser("counters")
    a.add_argument("db")
    a = sub.add_parser("traffic")
    a.add_argument("fetch_db")
    a.add_argument("write_db")
    a.add_argument("--kernel", required=True)
    a.add_argument("--tag", required=True)
    a.add_argument("--workload", required=True)
    a.add_argument("--copy-bytes", type=int, required=True)
    a.add_argument("--copy-kernel", default=COPY_KERNEL,
                   help="substring of the calibrating copy kernel's name")
    a.add_argument("--source", action="append", default=[])
    a.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    args = ap.parse_args(argv)
    if args.cmd == "kernels":
        print(kernel_table(args.db))
    elif args.cmd == "counters":
        for k, cs in sorted(counter_averages(args.db).items(), key=lambda kv: -kv[1]["avg_us"]):
            vals = " ".join(f"{c}={v:.4g}" for c, v in sorted(cs.items())
                            if c not in ("dispatches", "avg_us"))
            print(f"{k}: dispatches={cs['dispatches']} avg_us={cs['avg_us']:.2f} {vals}")
    else:
        rec = traffic(args.fetch_db, args.write_db, args.kernel, args.copy_bytes,
                      args.copy_kernel)
        rec["copy_kernel"] = args.copy_kernel
        rec["kernel"] = args.kernel
        rec["source_digest"] = source_digest(*args.source) if args.source else None
        rec["sources"] = args.source
        data = json.load(open(args.out)) if os.path.exists(args.out) else {}
        data[f"{args.tag}@{args.workload}"] = rec
        with open(args.out, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
        print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    sys.exit(main())
