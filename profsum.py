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
      sources the counters were taken with. Each DB may also be a JSON file
      written by `pmcdump`.

  python3 profsum.py pmcdump DB --out FILE.json
      per-kernel means of every counter of a `rocprofv3 --pmc` database (a
      few KB, where the database is tens of MB)

  python3 profsum.py sq COUNTERS --kernels PREFIX... --out profiles/NAME.md \
      --title T --cmd "C"
      VALU and MFMA busy fractions, waves per CU, wait fraction and MFMA
      flops per launch, from a run with GRBM_GUI_ACTIVE, SQ_WAVES,
      SQ_WAVE_CYCLES, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_VALU, SQ_INSTS_VALU,
      SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_F16
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


def counter_means(db):
    """{kernel name: {counter: [dispatches, mean value per dispatch]}} of a
    `rocprofv3 --pmc` database"""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
    agg = {}
    for n, c, v in rows:
        a = agg.setdefault(n, {}).setdefault(c, [0, 0.0])
        a[0] += 1
        a[1] += v
    return {n: {c: [a[0], a[1] / a[0]] for c, a in d.items()} for n, d in agg.items()}


def load_counters(path):
    """counter_means of a database, or the JSON file `pmcdump` wrote from one"""
    if path.endswith(".json"):
        return json.load(open(path))
    return counter_means(path)


def counter_per_kernel(path, counter):
    agg = {}
    for n, d in load_counters(path).items():
        if counter not in d:
            continue
        c, mean = d[counter]
        a = agg.setdefault(short_name(n), [0, 0.0])
        a[0] += c
        a[1] += mean * c
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
    entry = {"kernel": fk, "source_hash": a.source_hash or source_hash(),
             "bytes_per_launch": fetch_b + write_b,
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


def cmd_pmcdump(a):
    with open(a.out, "w") as fh:
        json.dump(counter_means(a.db), fh, indent=0)


# SQ counters -> fractions of the kernel's time. GRBM_GUI_ACTIVE counts GPU
# cycles once per XCD (8 of them); SQ_WAVE_CYCLES, SQ_ACTIVE_INST_VALU and
# SQ_WAIT_INST_ANY count in units of 4 cycles, summed over the chip;
# SQ_VALU_MFMA_BUSY_CYCLES counts busy cycles summed over the SIMDs; one unit
# of SQ_INSTS_VALU_MFMA_MOPS_F16 is 512 flops.
SIMDS, CUS, XCDS = 1024, 256, 8


def sq_row(c):
    g = c["GRBM_GUI_ACTIVE"][1] / XCDS
    simd_cycles = g * SIMDS
    waves = c["SQ_WAVES"][1]
    return {
        "launches": c["GRBM_GUI_ACTIVE"][0],
        "cycles": g,
        "valu_busy": c["SQ_ACTIVE_INST_VALU"][1] * 4 / simd_cycles,
        "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"][1] / simd_cycles,
        "waves_per_cu": c["SQ_WAVE_CYCLES"][1] * 4 / (g * CUS),
        "wait_frac": c["SQ_WAIT_INST_ANY"][1] / c["SQ_WAVE_CYCLES"][1],
        "mfma_gflop": c["SQ_INSTS_VALU_MFMA_MOPS_F16"][1] * 512 / 1e9,
        "valu_per_wave": c["SQ_INSTS_VALU"][1] / waves if waves else 0.0,
        "waves": waves,
    }


def cmd_sq(a):
    data = load_counters(a.counters)
    lines = [f"# {a.title}", "", "Command (from the repository root):", "", "```", a.cmd, "```", "",
             "Means per launch. VALU and MFMA busy are fractions of the SIMD cycles of the kernel "
             "(SQ_ACTIVE_INST_VALU x 4 and SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 x "
             "1024 SIMDs); waves per CU from SQ_WAVE_CYCLES x 4; wait is SQ_WAIT_INST_ANY / "
             "SQ_WAVE_CYCLES; flops are SQ_INSTS_VALU_MFMA_MOPS_F16 x 512.", "",
             "| kernel | launches | cycles per XCD | VALU busy | MFMA busy | waves per CU | wait "
             "| MFMA GFLOP | VALU instr per wave |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for prefix in a.kernels:
        hits = [(short_name(n), c) for n, c in data.items() if short_name(n).startswith(prefix)]
        if len(hits) != 1:
            sys.exit(f"expected one kernel named {prefix}..., found {[h[0] for h in hits]}")
        n, c = hits[0]
        r = sq_row(c)
        lines.append(f"| `{n}` | {r['launches']} | {r['cycles']:.0f} | {r['valu_busy']:.3f} | "
                     f"{r['mfma_busy']:.3f} | {r['waves_per_cu']:.2f} | {r['wait_frac']:.3f} | "
                     f"{r['mfma_gflop']:.1f} | {r['valu_per_wave']:.0f} |")
    if a.note:
        lines += ["", a.note]
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
    t.add_argument("--source-hash", default=None,
                   help="hash of the kernel sources the counters were taken with (default: "
                        "the sources in the tree now)")
    d = sub.add_parser("pmcdump")
    d.add_argument("db")
    d.add_argument("--out", required=True)
    q = sub.add_parser("sq")
    q.add_argument("counters")
    q.add_argument("--kernels", nargs="+", required=True)
    q.add_argument("--out", required=True)
    q.add_argument("--title", required=True)
    q.add_argument("--cmd", required=True)
    q.add_argument("--note", default="")
    a = p.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "pmcdump": cmd_pmcdump, "sq": cmd_sq}[a.what](a)


if __name__ == "__main__":
    main()
