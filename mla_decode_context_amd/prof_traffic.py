"""Turn rocprofv3 output of a bench.py run into the short summaries kept under profiles/.

Two subcommands:

  stats    DIR --kernel NAME[+NAME] --out FILE.md --cmd "..."
      Summarise ``*_kernel_stats.csv`` of a ``rocprofv3 --kernel-trace --stats``
      run: calls, average / min / max duration of every kernel.

  traffic  --fetch DIR --write DIR --copy-mib N --kernel NAME --workload W
           --alg-bytes B --cmd-fetch "..." --cmd-write "..." --out FILE.json
      HBM traffic per launch of kernel NAME from two ``--pmc`` runs (FETCH_SIZE,
      then WRITE_SIZE, both in KiB per dispatch), each scaled by what the same
      counter reads for the plain N-MiB copy that ``bench.py --copy-probe-mib N``
      runs first (the largest ``__amd_rocclr_copyBuffer`` dispatch).  The record
      carries the hash of the sources that build the kernel (``--sources``:
      decode16, h128 or merge); bench.py only reports it while that hash still
      matches.

Only reads CSV files; it touches no GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(_HERE))


def _csvs(d, suffix):
    out = sorted(set(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)))
    if not out:
        raise SystemExit(f"no *{suffix} under {d}")
    return out


def counter_per_dispatch(d, counter):
    """{dispatch_id: (kernel_name, value)} for one counter, summed over its rows."""
    res = {}
    for path in _csvs(d, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (path, r["Dispatch_Id"])
                name, v = res.get(key, (r["Kernel_Name"], 0.0))
                res[key] = (name, v + float(r["Counter_Value"]))
    return res


def kernel_average(rows, kernel):
    """Average per dispatch of each "+"-separated kernel name, summed: the
    traffic of one call that launches each of those kernels once."""
    tot, counts = 0.0, []
    for k in kernel.split("+"):
        vals = [v for name, v in rows.values() if k in name]
        if not vals:
            raise SystemExit(f"no dispatch of {k}")
        tot += sum(vals) / len(vals)
        counts.append(len(vals))
    return tot, min(counts)


def copy_reading(rows, expect_bytes):
    vals = [v for name, v in rows.values() if "copyBuffer" in name]
    if not vals:
        raise SystemExit("no copy dispatch found (run bench.py with --copy-probe-mib)")
    kib = max(vals)
    got = kib * 1024.0
    if not (0.5 * expect_bytes <= got <= 2.0 * expect_bytes):
        raise SystemExit(f"largest copy reads {got:.3g} B, expected about {expect_bytes:.3g} B")
    return kib


def cmd_traffic(a):
    from bench import DECODE16_SOURCES, H128_SOURCES, MERGE_SOURCES, kernel_source_hash

    sources = {"decode16": DECODE16_SOURCES, "h128": H128_SOURCES, "merge": MERGE_SOURCES}[a.sources]

    copy_bytes = a.copy_mib * (1 << 20)
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, "WRITE_SIZE")
    f_copy = copy_reading(fetch, copy_bytes)
    w_copy = copy_reading(write, copy_bytes)
    f_kib, nf = kernel_average(fetch, a.kernel)
    w_kib, nw = kernel_average(write, a.kernel)
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    fetch_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    rec = {
        "kernel": a.kernel,
        "workload": a.workload,
        "kernel_sources": sources,
        "kernel_source_hash": kernel_source_hash(sources),
        "bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes_per_launch": round(fetch_b),
        "write_bytes_per_launch": round(write_b),
        "alg_bytes_per_launch": a.alg_bytes,
        "traffic_over_alg": round((fetch_b + write_b) / a.alg_bytes, 4) if a.alg_bytes else None,
        "raw_fetch_kib_per_dispatch": round(f_kib, 1),
        "raw_write_kib_per_dispatch": round(w_kib, 1),
        "dispatches": {"fetch": nf, "write": nw},
        "copy_probe": {"bytes": copy_bytes, "fetch_kib": round(f_copy, 1), "write_kib": round(w_copy, 1),
                       "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5)},
        "commands": [a.cmd_fetch, a.cmd_write],
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def cmd_stats(a):
    rows = []
    for path in _csvs(a.dir, "kernel_stats.csv"):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel statistics: {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows[: a.top]:
        name = r["Name"].replace("|", "\\|")
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    if a.kernel:
        tot = 0.0
        for k in a.kernel.split("+"):
            sel = [r for r in rows if k in r["Name"]]
            if sel:
                r = sel[0]
                tot += float(r["AverageNs"])
                lines += ["", f"Kernel `{k}`: {r['Calls']} calls, average {float(r['AverageNs']) / 1e3:.2f} us."]
        if "+" in a.kernel:
            lines += ["", f"One call launches each of these once: {tot / 1e3:.2f} us per call in total."]
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="sub", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--kernel", default="")
    s.add_argument("--title", default="")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=12)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--sources", choices=["decode16", "h128", "merge"], default="decode16")
    t.add_argument("--alg-bytes", type=float, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    cmd_stats(a) if a.sub == "stats" else cmd_traffic(a)


if __name__ == "__main__":
    main()
