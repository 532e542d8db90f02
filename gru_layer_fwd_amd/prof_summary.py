"""Summarise rocprofv3 output of bench.py runs into short text files.

    python -m gru_layer_fwd_amd.prof_summary --workload NAME \
        --trace DIR/bench_kernel_trace.csv \
        [--fetch DIR/bench_counter_collection.csv --write DIR/bench_counter_collection.csv \
         --copy-bytes N] [--counters DIR/bench_counter_collection.csv ...] --command "..." --out profiles/NAME.md

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

def step_labels(names, dx_gemms=1):
    """Step of every dispatch, from the kernel names in dispatch order.
    `dx_gemms`: input-gradient products after each backward kernel (2 for
    bidirectional layers: one per direction, the second accumulating)."""
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
                lab = "dx_gemm" if gemms_after_bwd < dx_gemms else "dw_gemm"
                gemms_after_bwd += 1
            else:
                lab = "proj_gemm"
        elif "weight_transpose" in n:
            lab = "dx_gemm (W_ih transpose)" if phase == "after_bwd" else "rec_bwd (W_hh transpose)"
        elif "gather_transpose" in n:
            # after the backward kernel every transpose serves the weight
            # gradients (the gate gradients, x, h_{t-1})
            lab = "dw_gemm (transposes)" if phase == "after_bwd" else "aux"
        elif "dw_partials_finish" in n:
            lab = "dw_gemm (finish)"
        elif "gemm_finish" in n or "splitk_finish" in n or "rowsum_finish" in n or "rowsum_rows" in n:
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


def read_counters(path, dx_gemms=1):
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    labs = step_labels([r["Kernel_Name"] for r in rows], dx_gemms)
    per = collections.defaultdict(list)
    copies = []
    for r, lab in zip(rows, labs):
        v = float(r["Counter_Value"])
        if "copyBuffer" in r["Kernel_Name"]:
            copies.append(v)
        per[(r["Kernel_Name"], lab)].append(v)
    return per, (max(copies) if copies else None)


def read_counter_set(path, dx_gemms=1):
    """{(kernel, step): {counter: mean per dispatch}} from one --pmc pass with
    several counters (one row per dispatch and counter)."""
    by_disp = collections.OrderedDict()
    for r in sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"])):
        d = by_disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": {}})
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    names = [d["name"] for d in by_disp.values()]
    labs = step_labels(names, dx_gemms)
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for d, lab in zip(by_disp.values(), labs):
        for c, v in d["c"].items():
            acc[(d["name"], lab)][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def algorithmic_flops(workload):
    """Algorithmic FLOPs per launch of each layer step of a workload (the
    GEMM products; the persistent kernels' recurrent products)."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from gru_layer_fwd_amd import synth
    wl = synth.WORKLOADS[workload]
    G = 4 if wl.mode == "lstm" else 3
    TB, GH = wl.T * wl.B, G * wl.H
    return {"proj_gemm": 2.0 * TB * GH * wl.I, "dx_gemm": 2.0 * TB * GH * wl.I,
            "rec_fwd": 2.0 * TB * GH * wl.H, "rec_bwd": 2.0 * TB * GH * wl.H}


def counter_lines(sets, workload, cus=256, simds=4, xcds=8, dx_gemms=1):
    """Markdown for the MFMA and LDS counter passes. GRBM_GUI_ACTIVE counts
    the dispatch's cycles once per XCD (its sum over a dispatch is the
    duration times the clock times the XCD count); SQ_VALU_MFMA_BUSY_CYCLES
    sums the busy cycles of every SIMD (16 per 16x16x32 bf16 MFMA)."""
    lines = []
    alg = algorithmic_flops(workload)
    for path in sets:
        cs = read_counter_set(path, dx_gemms)
        counters = sorted({c for v in cs.values() for c in v})
        mops = [c for c in counters if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_")]
        lines += ["", f"Counters per dispatch ({', '.join(counters)}), mean over the dispatches of each kernel and step:", ""]
        head = ["kernel", "step"] + counters
        if "SQ_VALU_MFMA_BUSY_CYCLES" in counters and "GRBM_GUI_ACTIVE" in counters:
            head.append(f"MFMA busy % (busy / (GUI_ACTIVE / {xcds} XCDs x {cus} CUs x {simds} SIMDs))")
        if mops:
            head += ["MFMA FLOPs issued (512 x MOPS)", "algorithmic FLOPs", "issued / algorithmic"]
        if "SQ_LDS_BANK_CONFLICT" in counters and "SQ_ACTIVE_INST_LDS" in counters:
            head.append("LDS bank-conflict cycles / LDS active cycles")
        lines += ["| " + " | ".join(head) + " |", "|---" * len(head) + "|"]
        for (name, lab), v in sorted(cs.items(), key=lambda kv: kv[0][1]):
            if "copyBuffer" in name or "fillBuffer" in name:
                continue
            row = [f"`{short(name)}`", lab] + [f"{v.get(c, 0):.4g}" for c in counters]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in counters and "GRBM_GUI_ACTIVE" in counters:
                g = v.get("GRBM_GUI_ACTIVE", 0)
                row.append(f"{100 * v.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (g / xcds * cus * simds):.1f}" if g else "-")
            if mops:
                issued = 512.0 * sum(v.get(c, 0) for c in mops)
                a = alg.get(lab)
                row += [f"{issued:.4g}", f"{a:.4g}" if a else "-", f"{issued / a:.2f}" if a else "-"]
            if "SQ_LDS_BANK_CONFLICT" in counters and "SQ_ACTIVE_INST_LDS" in counters:
                act = v.get("SQ_ACTIVE_INST_LDS", 0)
                row.append(f"{v.get('SQ_LDS_BANK_CONFLICT', 0) / act:.3f}" if act else "-")
            lines.append("| " + " | ".join(row) + " |")
    return lines


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True, help="kernel_trace.csv of a --kernel-trace run")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--counters", action="append", default=[],
                    help="counter_collection.csv of a --pmc pass with several counters (MFMA, LDS); repeatable")
    ap.add_argument("--command", required=True, help="the command lines that produced the inputs")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json", default=None)
    ap.add_argument("--dx-gemms", type=int, default=1,
                    help="input-gradient products after each backward kernel (2 for bidirectional layers)")
    a = ap.parse_args(argv)

    rows = sorted(csv.DictReader(open(a.trace)), key=lambda r: int(r["Dispatch_Id"]))
    labs = step_labels([r["Kernel_Name"] for r in rows], a.dx_gemms)
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
        fetch, cf = read_counters(a.fetch, a.dx_gemms)
        write, cw = read_counters(a.write, a.dx_gemms)
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
    if a.counters:
        lines += counter_lines(a.counters, a.workload, dx_gemms=a.dx_gemms)
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
