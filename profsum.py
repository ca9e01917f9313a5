#!/usr/bin/env python3
"""Turns rocprofv3 output databases into the short text summaries kept under
profiles/ (this runs on any host; it reads the SQLite files rocprofv3 writes).

  python3 profsum.py stats DB --out profiles/NAME.md --title T --cmd "C"
      per-kernel call count and average / min / max / total duration
      (from a `rocprofv3 --kernel-trace --stats` run)

  python3 profsum.py traffic --config CFG --kernel PREFIX --fetch DB --write DB \
      --copy-fetch DB --copy-write DB --copy-bytes B --cmds "C1" "C2" "C3" "C4" \
      --out profiles/NAME.md
      HBM bytes per launch of the kernels whose name starts with PREFIX, from
      one FETCH_SIZE and one WRITE_SIZE pass, each scaled by what the same
      counter reads for one plain device copy of B bytes; recorded in
      profiles/hbm_traffic.json together with the hash of the expert kernel
      sources the counters were taken with.
"""
import argparse
import json
import os
import re
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def short_name(name):
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    depth, out = 0, []
    for ch in name:             # drop the argument list, keep template arguments
        if ch == "(" and depth == 0 and out:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).replace("void ", "").strip()


def kernel_rows(db):
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    name = "kernel_name" if "kernel_name" in cols else "name"
    return con.execute(f"select {name}, start, end from kernels").fetchall()


def stats(db):
    agg = {}
    for n, s, e in kernel_rows(db):
        a = agg.setdefault(short_name(n), [0, 0, float("inf"), 0])
        d = e - s
        a[0] += 1
        a[1] += d
        a[2] = min(a[2], d)
        a[3] = max(a[3], d)
    total = sum(a[1] for a in agg.values()) or 1
    return sorted(((n, a[0], a[1] / a[0] / 1e3, a[2] / 1e3, a[3] / 1e3, a[1] / 1e6,
                    100.0 * a[1] / total) for n, a in agg.items()), key=lambda r: -r[5])


def counter_per_kernel(db, counter):
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, value from counters_collection where counter_name=?",
                       (counter,)).fetchall()
    agg = {}
    for n, v in rows:
        a = agg.setdefault(short_name(n), [0, 0.0])
        a[0] += 1
        a[1] += v
    return {n: (c, s / c) for n, (c, s) in agg.items()}


def pick(per_kernel, prefix):
    hits = {n: v for n, v in per_kernel.items() if n.startswith(prefix)}
    if len(hits) != 1:
        sys.exit(f"expected one kernel named {prefix}..., found {sorted(hits)}")
    return next(iter(hits.items()))


def source_hash():
    sys.path.insert(0, ROOT)
    import bench
    return bench.kernel_source_hash()


def cmd_stats(a):
    rows = stats(a.db)
    lines = [f"# {a.title}", "", "Command (from the repository root):", "", "```", a.cmd, "```", "",
             "| calls | avg us | min us | max us | total ms | % | kernel |",
             "|---:|---:|---:|---:|---:|---:|---|"]
    for n, c, avg, mn, mx, tot, pct in rows:
        lines.append(f"| {c} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {tot:.3f} | {pct:.1f} | `{n}` |")
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(a):
    fk, (fc, fetch_kib) = pick(counter_per_kernel(a.fetch, "FETCH_SIZE"), a.kernel)
    wk, (wc, write_kib) = pick(counter_per_kernel(a.write, "WRITE_SIZE"), a.kernel)
    copy_prefix = "__amd_rocclr_copyBuffer"
    _, (_, cf_kib) = pick(counter_per_kernel(a.copy_fetch, "FETCH_SIZE"), copy_prefix)
    _, (_, cw_kib) = pick(counter_per_kernel(a.copy_write, "WRITE_SIZE"), copy_prefix)
    f_scale = a.copy_bytes / (cf_kib * 1024.0)
    w_scale = a.copy_bytes / (cw_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    entry = {"kernel": fk, "source_hash": source_hash(), "bytes_per_launch": fetch_b + write_b,
             "fetch_bytes": fetch_b, "write_bytes": write_b, "fetch_kib_raw": fetch_kib,
             "write_kib_raw": write_kib, "fetch_scale": f_scale, "write_scale": w_scale,
             "launches": [fc, wc]}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data.setdefault(a.config, {})[a.kernel] = entry
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    lines = [f"# HBM traffic of `{fk}` on {a.config}", "",
             "Commands (from the repository root): FETCH_SIZE and WRITE_SIZE over the "
             "workload, then the same two counters over one plain 1 GiB device copy:", "", "```"]
    lines += a.cmds + ["```", "",
                       f"| counter | raw KiB per launch | copy-calibrated scale | bytes per launch |",
                       "|---|---:|---:|---:|",
                       f"| FETCH_SIZE | {fetch_kib:.2f} | {f_scale:.5f} | {fetch_b:.0f} |",
                       f"| WRITE_SIZE | {write_kib:.2f} | {w_scale:.5f} | {write_b:.0f} |",
                       f"| total | | | {fetch_b + write_b:.0f} |", "",
                       f"Launches averaged: {fc} (fetch pass), {wc} (write pass). "
                       f"Copy kernel: {cf_kib:.2f} KiB fetched and {cw_kib:.2f} KiB written "
                       f"for {a.copy_bytes} bytes each way. Expert kernel source hash "
                       f"{entry['source_hash']}."]
    if a.algorithmic:
        lines.append(f"Algorithmic bytes per launch: {a.algorithmic:.0f}; measured / algorithmic "
                     f"= {(fetch_b + write_b) / a.algorithmic:.3f}.")
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("db")
    s.add_argument("--out", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    for k in ("config", "kernel", "fetch", "write", "copy_fetch", "copy_write", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    t.add_argument("--algorithmic", type=float, default=None)
    t.add_argument("--cmds", nargs=4, required=True)
    a = p.parse_args()
    cmd_stats(a) if a.what == "stats" else cmd_traffic(a)


if __name__ == "__main__":
    main()
