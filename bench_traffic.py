"""Turn two rocprofv3 counter runs of bench.py into per-launch HBM traffic.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o run -- \\
        python3 bench.py --steps 3 --warmup 1 --profile-steps 1 --no-cpu-baseline --no-decode \\
        --no-configs --no-clock --copy-probe-mib 1024
    rocprofv3 --pmc WRITE_SIZE ... (same command, another directory)
    python bench_traffic.py <dir_f>/run_counter_collection.csv <dir_w>/run_counter_collection.csv \\
        --copy-mib 1024 --json profiles/traffic.json --md profiles/traffic_d12_bench.md
    python bench_traffic.py --stats <dir>/<name>_kernel_stats.csv   (markdown table of a --stats run)

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  The copy probe
moves a known number of bytes (read once, written once), so the ratio of its
known size to its measured counters calibrates both; each kernel's average
counter per dispatch is multiplied by that factor.  profiles/traffic.json keeps,
per kernel, the calibrated bytes per launch and a hash of the kernel's source, so
bench.py reports the figure only while the kernel is unchanged.
"""

from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

from bench import KERNEL_SOURCES, kernel_source_hash

SHORT = {  # kernel symbol fragment -> bench's kernel name
    "attn_fwd_bf16_kernel": "fwd",
    "bwd_dkdv_kernel": "bwd_dkdv",
    "bwd_dq_kernel": "bwd_dq",
    "bwd_delta_kernel": "bwd_delta",
    "qknorm_rope_kernel": "qknorm_rope",
    "decode_split_kernel": "decode_split",
}


def per_kernel(path, counter):
    vals = collections.defaultdict(list)
    copy = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        for frag, short in SHORT.items():
            if frag in name:
                vals[short].append(v)
                break
        else:
            if re.search(r"copyBuffer|copy", name, re.I):
                copy.append(v)
    return vals, copy


def stats_table(path):
    """Markdown table of a rocprofv3 --stats kernel summary (durations in us)."""
    rows = ["| kernel | calls | total us | average us | min us | max us | share |", "|---|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(path)):
        name = r["Name"]
        m = re.search(r"(\w+_kernel(<[^>]*>)?)", name)
        short = m.group(1) if m else name[:48]
        rows.append(f"| {short} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                    f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                    f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(rows)


def main():
    if len(sys.argv) >= 3 and sys.argv[1] == "--stats":
        print(stats_table(sys.argv[2]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--json", default="profiles/traffic.json")
    ap.add_argument("--md", default=None)
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    fetch, fcopy = per_kernel(a.fetch_csv, "FETCH_SIZE")
    write, wcopy = per_kernel(a.write_csv, "WRITE_SIZE")
    if not fcopy or not wcopy:
        sys.exit("no copy-probe dispatch found in the counter files")
    known_kib = a.copy_mib * 1024.0
    # the largest copy dispatches are the probe's (input set-up copies are smaller)
    f_meas = max(fcopy)
    w_meas = max(wcopy)
    kf, kw = known_kib / f_meas, known_kib / w_meas
    out = {"copy_probe_mib": a.copy_mib, "copy_fetch_kib": f_meas, "copy_write_kib": w_meas,
           "fetch_factor": kf, "write_factor": kw, "command": a.command, "kernels": {}}
    lines = ["| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | calibrated MB/launch (read + write) |",
             "|---|---|---|---|---|"]
    for k in sorted(set(fetch) | set(write)):
        if not fetch.get(k) or not write.get(k):
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        nbytes = (fk * kf + wk * kw) * 1024.0
        out["kernels"][k] = {"fetch_kib": fk, "write_kib": wk, "bytes_per_launch": round(nbytes),
                             "dispatches": len(fetch[k]), "source_hash": kernel_source_hash(KERNEL_SOURCES[k])}
        lines.append(f"| {k} | {len(fetch[k])} | {fk:.0f} | {wk:.0f} | {nbytes / 1e6:.1f} |")
    os.makedirs(os.path.dirname(a.json) or ".", exist_ok=True)
    json.dump(out, open(a.json, "w"), indent=1)
    md = [f"Calibration: a {a.copy_mib} MiB device copy read {f_meas:.0f} KiB and wrote {w_meas:.0f} KiB "
          f"(factors {kf:.3f} and {kw:.3f}).", ""] + lines
    text = "\n".join(md)
    print(text)
    if a.md:
        with open(a.md, "w") as fh:
            fh.write("# HBM traffic per launch, d12 bench step (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n")
            if a.command:
                fh.write("Commands:\n\n" + "\n".join("    " + c for c in a.command.split(" ;; ")) + "\n\n")
            fh.write(text + "\n")


if __name__ == "__main__":
    main()
