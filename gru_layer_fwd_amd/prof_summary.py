"""Summarise rocprofv3 output of bench.py runs into short text files.

    python -m gru_layer_fwd_amd.prof_summary --workload NAME \
        --stats DIR/bench_kernel_stats.csv \
        [--fetch DIR/bench_counter_collection.csv --write DIR/bench_counter_collection.csv \
         --copy-bytes N] --command "..." --out profiles/NAME.md

Writes a markdown table of per-kernel durations (kernel-trace --stats) and,
when the two counter passes are given, HBM bytes per launch from FETCH_SIZE
and WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the
reading of the calibration copy (the largest __amd_rocclr_copyBuffer
dispatch, `copy-bytes` read and as many written) equal to its true size. The
per-launch bytes of every layer kernel are also merged into
profiles/traffic.json under the current kernel-source hash, which bench.py
reports only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import sys

LABELS = (("rec_fwd", "rec_fwd"), ("rec_bwd", "rec_bwd"), ("gemm_kernelIDF16bLb0ELb0E", "proj_gemm"),
          ("gemm_kernelIfLb0ELb0E", "proj_gemm"), ("gemm_kernelIDF16bLb0ELb1E", "dx_gemm"),
          ("gemm_kernelIfLb0ELb1E", "dx_gemm"), ("gemm_kernel<bool", "dw_gemm"), ("gemm_kernelIDF16bLb1ELb1E", "dw_gemm"),
          ("gemm_kernelIfLb1ELb1E", "dw_gemm"), ("colsum", "db_colsum"), ("fill", "fill"),
          ("lstm_cell_scan", "aux"), ("zero_inactive", "aux"), ("gather_first_rows", "aux"), ("att_reduce", "aux"))


def label_of(name: str) -> str:
    for key, lab in LABELS:
        if key in name:
            return lab
    return "other"


def short(name: str) -> str:
    return name if len(name) <= 90 else name[:87] + "..."


def read_counters(path):
    rows = list(csv.DictReader(open(path)))
    per = collections.defaultdict(list)
    copies = []
    for r in rows:
        v = float(r["Counter_Value"])
        if "copyBuffer" in r["Kernel_Name"]:
            copies.append(v)
        per[r["Kernel_Name"]].append(v)
    return per, (max(copies) if copies else None)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--command", required=True, help="the command lines that produced the inputs")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json", default=None)
    a = ap.parse_args(argv)

    stats = list(csv.DictReader(open(a.stats)))
    lines = [f"# rocprofv3 kernel summary: {a.workload}", "", "Produced by:", "", "```"]
    lines += a.command.strip().splitlines() + ["```", ""]
    lines += ["| kernel | step | calls | avg us | total % |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{short(r['Name'])}` | {label_of(r['Name'])} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    traffic = {}
    if a.fetch and a.write and a.copy_bytes:
        fetch, cf = read_counters(a.fetch)
        write, cw = read_counters(a.write)
        kib = a.copy_bytes / 1024.0
        f_scale, w_scale = kib / cf, kib / cw
        lines += ["", f"HBM traffic per launch (FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}; factors make "
                  f"the {a.copy_bytes >> 20} MiB calibration copy read and write exactly its size):", "",
                  "| kernel | step | read MiB | write MiB | total MiB |", "|---|---|---|---|---|"]
        for k in fetch:
            if "copyBuffer" in k or k not in write:
                continue
            fr = sum(fetch[k]) / len(fetch[k]) * f_scale * 1024
            wr = sum(write[k]) / len(write[k]) * w_scale * 1024
            lab = label_of(k)
            lines.append(f"| `{short(k)}` | {lab} | {fr / 2**20:.1f} | {wr / 2**20:.1f} | {(fr + wr) / 2**20:.1f} |")
            if lab in ("rec_fwd", "rec_bwd", "proj_gemm", "dx_gemm"):
                traffic[lab] = fr + wr
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if traffic:
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        path = a.traffic_json or os.path.join(os.path.dirname(os.path.abspath(a.out)), "traffic.json")
        try:
            t = json.load(open(path))
        except (OSError, ValueError):
            t = {}
        h = bench.kernel_hash()
        for lab, b in traffic.items():
            t.setdefault(a.workload, {})[lab] = {"bytes_per_launch": b, "kernel_hash": h}
        with open(path, "w") as fh:
            json.dump(t, fh, indent=1, sort_keys=True)
    print(f"wrote {a.out}")


if __name__ == "__main__":
    main()
