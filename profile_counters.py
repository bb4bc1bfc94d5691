#!/usr/bin/env python3
"""Turn rocprofv3 output of bench.py runs into the short summaries kept in profiles/.

    # kernel durations (rocprofv3 --kernel-trace --stats --output-format csv)
    python profile_counters.py trace <run dir> --workload target --command "<command>" > profiles/<name>.md

    # instruction counters of the attention kernel (one or more --pmc runs)
    python profile_counters.py sq <run dir> [<run dir> ...] --workload target --command "<command>" ... \
        > profiles/<name>.md

    # HBM traffic of the attention kernel from two counter runs of
    #   bench.py --calibrate-copy  (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)
    python profile_counters.py counters --fetch <run dir> --write <run dir> --workload target \\
        --command-fetch "<command>" --command-write "<command>"

FETCH_SIZE and WRITE_SIZE count KiB per dispatch at the L2/memory interface.
Each is scaled by bytes / counter for the calibration copy (a plain
elementwise kernel that reads and writes exactly COPY_BYTES each), so the
figure is in bytes of the same kind as the algorithmic bytes.  The JSON
record carries the attention kernel's source hash; bench.py reports the
traffic only while that hash still matches the sources.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

ATTN = "attn_fwd_kernel"
COPY = "neg_kernel"


def _find(run_dir: str, suffix: str) -> list[str]:
    files = sorted(glob.glob(os.path.join(run_dir, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {run_dir}")
    return files


def _short(name: str) -> str:
    name = name.replace("sage::(anonymous namespace)::", "")
    if COPY in name:
        return "torch neg (calibration copy)"
    return name.split("(")[0] if "(" in name and "<" not in name.split("(")[0] else name[:90]


def trace(args):
    rows = []
    for f in _find(args.run_dir, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    print(f"# Kernel durations: {args.workload}\n")
    print("Command (repository root, one MI355X):\n")
    print(f"    {args.command}\n")
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{100 * float(r['TotalDurationNs']) / tot:.1f}% |")


def _per_dispatch(run_dir: str, counter: str) -> dict[str, float]:
    """Mean counter value per dispatch, by kernel name."""
    acc: dict[tuple[str, str], float] = {}
    for f in _find(run_dir, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
                acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel: dict[str, list[float]] = {}
    for (name, _), v in acc.items():
        by_kernel.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in by_kernel.items()}


def _pick(table: dict[str, float], needle: str) -> float:
    hits = [v for k, v in table.items() if needle in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {needle!r}, found {len(hits)}")
    return hits[0]


def counters(args):
    from bench import COPY_BYTES, kernel_source_hash
    fetch = _per_dispatch(args.fetch, "FETCH_SIZE")
    write = _per_dispatch(args.write, "WRITE_SIZE")
    a_f, c_f = _pick(fetch, ATTN), _pick(fetch, COPY)
    a_w, c_w = _pick(write, ATTN), _pick(write, COPY)
    f_scale = COPY_BYTES / c_f          # bytes per counter unit, read side
    w_scale = COPY_BYTES / c_w          # bytes per counter unit, write side
    rec = {
        "workload": args.workload,
        "kernel": ATTN,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_size_per_dispatch": a_f,
        "write_size_per_dispatch": a_w,
        "copy_bytes": COPY_BYTES,
        "copy_fetch_size": c_f,
        "copy_write_size": c_w,
        "bytes_per_fetch_unit": f_scale,
        "bytes_per_write_unit": w_scale,
        "hbm_read_bytes_per_launch": a_f * f_scale,
        "hbm_write_bytes_per_launch": a_w * w_scale,
        "hbm_bytes_per_launch": a_f * f_scale + a_w * w_scale,
        "command_fetch": args.command_fetch,
        "command_write": args.command_write,
    }
    out = os.path.join(ROOT, "profiles", "attn_fwd_counters.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def _tile_waves(w) -> int:
    """Wave-tiles of the attention kernel: 4 waves per 128-query block, one per 128-key tile it visits."""
    nblk = -(-w.N // 128)
    if w.causal:
        tiles = sum(-(-min(w.N, 128 * (qb + 1)) // 128) for qb in range(nblk))
    else:
        tiles = nblk * nblk
    return w.B * w.H * 4 * tiles


def sq(args):
    from quantized_attention_sage_amd.workloads import WORKLOADS
    w = WORKLOADS[args.workload]
    tw = _tile_waves(w)
    rows = []
    for run_dir, cmd in zip(args.run_dirs, args.command):
        names = set()
        for f in _find(run_dir, "counter_collection.csv"):
            with open(f) as fh:
                names |= {r["Counter_Name"] for r in csv.DictReader(fh)}
        for name in sorted(names):
            rows.append((name, _pick(_per_dispatch(run_dir, name), args.kernel), cmd))
    print(f"# Instruction counters of {args.kernel}: {args.workload}\n")
    print(f"Per dispatch (mean over the dispatches of the run); a wave-tile is one wave's share (32 queries) "
          f"of one 128-key tile, {tw} per dispatch here.\n")
    print("Commands (repository root, one MI355X):\n")
    for cmd in args.command:
        print(f"    {cmd}\n")
    print("| counter | per dispatch | per wave-tile |")
    print("|---|---|---|")
    for name, v, _ in rows:
        print(f"| {name} | {v:.6g} | {v / tw:.4g} |")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("run_dir")
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    q = sub.add_parser("sq")
    q.add_argument("run_dirs", nargs="+")
    q.add_argument("--workload", required=True)
    q.add_argument("--command", required=True, action="append")
    q.add_argument("--kernel", default=ATTN, help="kernel name to report (default attn_fwd_kernel)")
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    args = ap.parse_args()
    {"trace": trace, "sq": sq, "counters": counters}[args.cmd](args)


if __name__ == "__main__":
    main()
