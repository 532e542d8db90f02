"""Summarise rocprofv3 output of bench.py runs into short text files.

    python -m gru_layer_fwd_amd.prof_summary --workload NAME \
        --trace DIR/bench_kernel_trace.csv \
        [--fetch DIR/bench_counter_collection.csv --write DIR/bench_counter_collection.csv \
         --copy-bytes N] --command "..." --out profiles/NAME.md

Writes a markdown table of per-kernel durations (from the kernel trace) and,
when the two counter passes are given, HBM bytes per launch from FETCH_SIZE
and WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the
reading of the calibration copy (the largest __amd_rocclr_copyBuffer
dispatch, `copy-bytes` read and as many written) equal to its true size. The
per-launch bytes of every layer kernel are also merged into
profiles/traffic.json under the current kernel-source hash, which bench.py
reports only while the sources are unchanged.

One GEMM kernel can serve several steps of the layer (the input projection
and the input gradient share an instantiation), so each dispatch is given
the step it performs from its place in the dispatch order: GEMMs before the
forward recurrence are the projection; after the backward recurrence the
first GEMM is the input gradient and the later ones the weight gradients;
transposes and finishing passes go with the step they serve (a weight
transpose before the backward recurrence is W_hh's, one after it W_ih's).
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import sys

def step_labels(names):
    """Step of every dispatch, from the kernel names in dispatch order."""
    out, phase, gemms_after_bwd = [], "start", 0
    for n in names:
        if "rec_fwd" in n:
            lab, phase = "rec_fwd", "after_fwd"
        elif "rec_bwd" in n:
            lab, phase, gemms_after_bwd = "rec_bwd", "after_bwd", 0
        elif "fill_i32" in n:
            lab = "fill"
            if phase == "after_bwd":
                phase = "start"
        elif "gemm_kernel" in n:
            if phase == "after_bwd":
                lab = "dx_gemm" if gemms_after_bwd == 0 else "dw_gemm"
                gemms_after_bwd += 1
            else:
                lab = "proj_gemm"
        elif "weight_transpose" in n:
            lab = "dx_gemm (W_ih transpose)" if phase == "after_bwd" else "rec_bwd (W_hh transpose)"
        elif "gather_transpose" in n:
            lab = "dw_gemm (transposes)" if phase == "after_bwd" else "aux"
        elif "splitk_finish" in n or "rowsum_finish" in n or "rowsum_rows" in n:
            lab = "dw_gemm (finish)" if phase == "after_bwd" else "proj_gemm (finish)"
        elif "colsum" in n:
            lab = "db_colsum"
        elif "copyBuffer" in n or "fillBuffer" in n:
            lab = "other"
        else:
            lab = "aux"
        out.append(lab)
    return out


def short(name: str) -> str:
    return name if len(name) <= 90 else name[:87] + "..."


def read_counters(path):
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    labs = step_labels([r["Kernel_Name"] for r in rows])
    per = collections.defaultdict(list)
    copies = []
    for r, lab in zip(rows, labs):
        v = float(r["Counter_Value"])
        if "copyBuffer" in r["Kernel_Name"]:
            copies.append(v)
        per[(r["Kernel_Name"], lab)].append(v)
    return per, (max(copies) if copies else None)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True, help="kernel_trace.csv of a --kernel-trace run")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--command", required=True, help="the command lines that produced the inputs")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json", default=None)
    a = ap.parse_args(argv)

    rows = sorted(csv.DictReader(open(a.trace)), key=lambda r: int(r["Dispatch_Id"]))
    labs = step_labels([r["Kernel_Name"] for r in rows])
    dur = collections.defaultdict(list)
    for r, lab in zip(rows, labs):
        dur[(r["Kernel_Name"], lab)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in dur.values())
    lines = [f"# rocprofv3 kernel summary: {a.workload}", "", "Produced by:", "", "```"]
    lines += a.command.strip().splitlines() + ["```", ""]
    lines += ["| kernel | step | calls | avg us | total % |", "|---|---|---|---|---|"]
    for (name, lab), v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{short(name)}` | {lab} | {len(v)} | {sum(v) / len(v):.1f} | {100 * sum(v) / total:.2f} |")
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
            name, lab = k
            if "copyBuffer" in name or k not in write:
                continue
            fr = sum(fetch[k]) / len(fetch[k]) * f_scale * 1024
            wr = sum(write[k]) / len(write[k]) * w_scale * 1024
            lines.append(f"| `{short(name)}` | {lab} | {fr / 2**20:.1f} | {wr / 2**20:.1f} | {(fr + wr) / 2**20:.1f} |")
            if lab in ("rec_fwd", "rec_bwd", "proj_gemm", "dx_gemm", "dw_gemm"):
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
