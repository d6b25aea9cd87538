"""Summaries of rocprofv3 runs of bench.py: HBM traffic per launch, MFMA counters
and kernel-trace statistics, per kernel and workload.

    cd /tmp && export TMPDIR=/tmp
    B="python3 <repo>/bench.py --steps 2 --warmup 1 --profile-steps 1 --no-cpu-baseline --no-configs --no-clock --decode-iters 4"
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <f> -o run -- $B --copy-probe-mib 1024
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <w> -o run -- $B --copy-probe-mib 1024
    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU \\
        SQ_INSTS_LDS SQ_INSTS_MFMA SQ_WAVE_CYCLES SQ_INSTS_SALU GRBM_GUI_ACTIVE --output-format csv -d <m> -o run -- $B
    rocprofv3 --kernel-trace --stats --output-format csv -d <t> -o bench -- python3 <repo>/bench.py \\
        --no-cpu-baseline --no-configs --no-clock

    python bench_traffic.py traffic <f>/run_counter_collection.csv <w>/run_counter_collection.csv \\
        --copy-mib 1024 --json profiles/traffic.json --md profiles/traffic_gqa_step_and_decode.md
    python bench_traffic.py mfma <m>/run_counter_collection.csv --md profiles/mfma_gqa_step.md
    python bench_traffic.py stats <t>/bench_kernel_stats.csv

Dispatches are grouped by kernel and grid size, and each group is labelled with
the workload whose launch has that grid (the bench's default step is the
grouped-query layer; its decode runs the engine-decode batch at two windows, and
each decode_combine belongs to the decode_split launched just before it).
FETCH_SIZE and WRITE_SIZE are KiB per dispatch; the copy probe moves a known
number of bytes (read once, written once), so the ratio of its size to its
counters calibrates both.  profiles/traffic.json keeps, per workload and kernel,
the calibrated bytes per launch and a hash of the kernel's source, so bench.py
reports a figure only while the kernel is unchanged.  GRBM_GUI_ACTIVE is summed
over the XCDs; MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE /
XCDs x SIMDs).
"""

from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from bench import KERNEL_SOURCES, kernel_source_hash  # noqa: E402

SHORT = {  # kernel symbol -> bench's kernel name
    "attn_fwd_bf16_kernel": "fwd",
    "bwd_dkdv_kernel": "bwd_dkdv",
    "bwd_dq_kernel": "bwd_dq",
    "bwd_delta_kernel": "bwd_delta",
    "qknorm_rope_kernel": "qknorm_rope",
    "decode_split_kernel": "decode_split",
    "decode_combine_kernel": "decode_combine",
    "prefill_append_kernel": "prefill_append",
    "cache_replicate_kernel": "cache_replicate",
}
N_XCD, N_SIMD = 8, 1024


def short_name(full):
    m = re.search(r"(\w+_kernel)(<[^>]*>)?\(", full)
    if m:
        return SHORT.get(m.group(1), m.group(1))
    return "copy" if "copyBuffer" in full else full[:40]


def grid_labels():
    """(kernel, grid size in threads) -> workload label, from the workload shapes."""
    from workloads import D12, DECODE, GQA, PREFILL
    lab = {}
    for cfg in (GQA, D12):
        B, T, H, KV = cfg.B, cfg.T, cfg.H, cfg.KV
        for k, g in (("fwd", -(-T // 128) * B * H * 256), ("bwd_dq", -(-T // 128) * B * H * 256),
                     ("bwd_dkdv", -(-T // 128) * B * KV * 256), ("bwd_delta", -(-(B * T * H) // 64) * 256),
                     ("qknorm_rope", None)):
            if g is not None:
                lab.setdefault((k, g), cfg.name)
    c = DECODE
    for W in c.windows:
        span = c.T_max if W < 0 or W + 1 > c.T_max else W + 1
        lab[("decode_split", c.B * c.KV * (-(-span // 128)) * 256)] = f"{c.name} W={W}"
    p = PREFILL
    lab[("fwd", -(-p.Tn // 128) * p.B * p.H * 256)] = p.name
    return lab


def dispatches(path):
    """Rows of a counter csv as dispatch records {id, kernel, grid, counters{}} in dispatch order."""
    by_id = {}
    for r in csv.DictReader(open(path)):
        d = by_id.setdefault(int(r["Dispatch_Id"]), {"id": int(r["Dispatch_Id"]), "kernel": short_name(r["Kernel_Name"]),
                                                     "grid": int(r["Grid_Size"]), "c": {}})
        d["c"][r["Counter_Name"]] = float(r["Counter_Value"])
    out = sorted(by_id.values(), key=lambda d: d["id"])
    lab = grid_labels()
    last_split = None
    for d in out:
        d["label"] = lab.get((d["kernel"], d["grid"]))
        if d["kernel"] == "decode_split":
            last_split = d["label"]
        elif d["kernel"] == "decode_combine":
            d["label"] = last_split
    return out


def grouped(ds):
    g = collections.defaultdict(list)
    for d in ds:
        if d["label"] is not None:
            g[(d["label"], d["kernel"])].append(d)
    return g


def cmd_traffic(a):
    fd, wd = dispatches(a.fetch_csv), dispatches(a.write_csv)
    fcopy = [d["c"]["FETCH_SIZE"] for d in fd if d["kernel"] == "copy"]
    wcopy = [d["c"]["WRITE_SIZE"] for d in wd if d["kernel"] == "copy"]
    if not fcopy or not wcopy:
        sys.exit("no copy-probe dispatch found in the counter files")
    known_kib = a.copy_mib * 1024.0
    f_meas, w_meas = fcopy[-1], wcopy[-1]  # the probe's copies are the run's last dispatches
    kf, kw = known_kib / f_meas, known_kib / w_meas
    out = {"copy_probe_mib": a.copy_mib, "copy_fetch_kib": f_meas, "copy_write_kib": w_meas, "fetch_factor": kf,
           "write_factor": kw, "workloads": {}}
    lines = ["| workload | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated MB per launch (read + write) |",
             "|---|---|---|---|---|---|"]
    gf, gw = grouped(fd), grouped(wd)
    for key in sorted(set(gf) & set(gw)):
        label, k = key
        if k not in KERNEL_SOURCES:
            continue
        fk = sum(d["c"]["FETCH_SIZE"] for d in gf[key]) / len(gf[key])
        wk = sum(d["c"]["WRITE_SIZE"] for d in gw[key]) / len(gw[key])
        nbytes = (fk * kf + wk * kw) * 1024.0
        out["workloads"].setdefault(label, {"kernels": {}})["kernels"][k] = {
            "fetch_kib": fk, "write_kib": wk, "bytes_per_launch": round(nbytes), "read_bytes": round(fk * kf * 1024),
            "write_bytes": round(wk * kw * 1024), "dispatches": len(gf[key]),
            "source_hash": kernel_source_hash(KERNEL_SOURCES[k])}
        lines.append(f"| {label} | {k} | {len(gf[key])} | {fk:.0f} | {wk:.0f} | {nbytes / 1e6:.1f} "
                     f"({fk * kf * 1024 / 1e6:.1f} + {wk * kw * 1024 / 1e6:.1f}) |")
    json.dump(out, open(a.json, "w"), indent=1)
    text = "\n".join([f"Calibration: a {a.copy_mib} MiB device copy read {f_meas:.0f} KiB and wrote {w_meas:.0f} KiB "
                      f"(factors {kf:.3f} and {kw:.3f}).", ""] + lines)
    print(text)
    if a.md:
        with open(a.md, "w") as fh:
            fh.write(a.title + "\n\n")
            if a.command:
                fh.write("Commands (from /tmp, TMPDIR=/tmp):\n\n" + "\n".join("    " + c for c in a.command.split(" ;; "))
                         + "\n\n")
            fh.write(text + "\n")


def cmd_mfma(a):
    ds = dispatches(a.csv)
    lines = ["| workload | kernel | dispatches | MFMA GFLOP per launch (MOPS_BF16 x 512) | MFMA busy | "
             "MFMA / VALU / LDS / SALU instructions per launch (M) | wave-cycles per launch (G) |",
             "|---|---|---|---|---|---|---|"]
    out = {}
    for (label, k), group in sorted(grouped(ds).items()):
        n = len(group)
        avg = {c: sum(d["c"].get(c, 0.0) for d in group) / n for c in group[0]["c"]}
        fl = avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        gui = avg.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        util = avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * N_SIMD) if gui else 0.0
        out.setdefault(label, {})[k] = {"mfma_flop": fl, "mfma_busy": util, "dispatches": n,
                                        **{c: v for c, v in avg.items()}}
        lines.append(f"| {label} | {k} | {n} | {fl / 1e9:.1f} | {100 * util:.1f}% | "
                     f"{avg.get('SQ_INSTS_MFMA', 0) / 1e6:.2f} / {avg.get('SQ_INSTS_VALU', 0) / 1e6:.1f} / "
                     f"{avg.get('SQ_INSTS_LDS', 0) / 1e6:.1f} / {avg.get('SQ_INSTS_SALU', 0) / 1e6:.1f} | "
                     f"{avg.get('SQ_WAVE_CYCLES', 0) / 1e9:.2f} |")
    text = "\n".join(lines)
    print(text)
    if a.json:
        json.dump(out, open(a.json, "w"), indent=1)
    if a.md:
        with open(a.md, "w") as fh:
            fh.write(a.title + "\n\n")
            if a.command:
                fh.write("Command (from /tmp, TMPDIR=/tmp):\n\n    " + a.command + "\n\n")
            fh.write(f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} XCDs x {N_SIMD} SIMDs); "
                     "GRBM_GUI_ACTIVE is reported summed over the XCDs.\n\n")
            fh.write(text + "\n")


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
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    t.add_argument("--md", default=None)
    t.add_argument("--title", default="# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    t.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--json", default=None)
    m.add_argument("--md", default=None)
    m.add_argument("--title", default="# MFMA counters per launch (rocprofv3)")
    m.add_argument("--command", default="")
    s = sub.add_parser("stats")
    s.add_argument("csv")
    a = ap.parse_args()
    if a.cmd == "traffic":
        cmd_traffic(a)
    elif a.cmd == "mfma":
        cmd_mfma(a)
    else:
        print(stats_table(a.csv))


if __name__ == "__main__":
    main()
