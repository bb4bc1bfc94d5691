#!/usr/bin/env python3
"""Throughput of the quantized attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload target] [--gpus 1]

One step = sage_quant_qk + sage_quant_v + sage_attn_fwd over one batch of
synthetic inputs already resident in HBM.  Prints ONE JSON line.  `value` is
attention TOPS of the whole step: 4*B*H*N^2*d (halved when causal) divided by
the step time.  `roofline` covers the attention kernel, timed with HIP events
on the stream it is launched on.  `cpu_baseline` times the CPU oracle
(quantisation emulation plus tiled attention emulation) on a bounded sample of
the same workload and extrapolates per head.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS = 5000.0      # MI355X dense INT8 and FP8 matrix peak (both 5.0 P/s)
PEAK_BF16_TOPS = 2500.0 # MI355X dense bf16 / fp16 matrix peak
# With the 16-bit P~V half of the work (QK^T) runs at the INT8 rate and half
# (P~V) at the bf16 rate: the path's peak is 2 / (1/5000 + 1/2500) TOPS.
PEAK_PV16_TOPS = 2.0 / (1.0 / PEAK_TOPS + 1.0 / PEAK_BF16_TOPS)
PEAK_FP4_TOPS = 10100.0 # MI355X dense FP4 and FP6 matrix peak
# With MXFP4 Q and K, QK^T runs at the FP4 rate and P~V at the FP8 one.
PEAK_MXFP4_TOPS = 2.0 / (1.0 / PEAK_FP4_TOPS + 1.0 / PEAK_TOPS)
HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 30    # calibration copy: reads and writes this many bytes
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E


def quant_bytes(w, pv: str = "fp8", qk_format: str = "int") -> tuple[int, int]:
    """Algorithmic HBM bytes of sage_quant_qk and sage_quant_v.

    quant_qk reads Q and K once (2 B/pos each), writes their int8 codes over
    the padded length (1 B/pos each) and the bias (4 B per query block and
    key; MXFP4 codes are 0.5 B/pos plus a scale byte per 32); quant_v reads V
    once and writes its FP8 codes (with the 16-bit P~V, V itself in the
    kernel's layout, 2 B/pos).  Scales and means (below 0.1
    B/pos) are left out, and so are the re-reads of the statistic passes."""
    n_pad = -(-w.N // 128) * 128
    bh = w.B * w.H
    pos, pos_pad = bh * w.N * w.d, bh * n_pad * w.d
    codes = 2 * (pos_pad // 2 + pos_pad // 32) if qk_format == "mxfp4" else 2 * pos_pad
    qk = 4 * pos + codes + bh * (n_pad // 128) * n_pad * 4
    v = 2 * pos + pos_pad * (2 if pv == "f16" else 1)
    return qk, v
COUNTERS = os.path.join(ROOT, "profiles", "attn_fwd_counters.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("attn.hip", "sage_internal.h"):
        with open(os.path.join(ROOT, "quantized_attention_sage_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel changed since."""
    try:
        with open(COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, sample_blocks: int = 96, pv: str = "fp8", qk_format: str = "int"):
    """Time the oracle on one head: quantisation of the head plus the tiled
    emulation of `sample_blocks` query blocks, extrapolated to the workload."""
    import numpy as np
    import oracle
    from oracle.quant import QuantParams
    from quantized_attention_sage_amd.workloads import make_inputs, scaled

    one = scaled(w, B=1, H=1)
    q, k, v = make_inputs(one)
    p = QuantParams(qk_bits=w.qk_bits, gran=w.gran, pv=w.dtype if pv == "f16" else "fp8", qk_format=qk_format)
    t0 = time.perf_counter()
    qk = oracle.quant_qk(q, k, p, with_bias=False)
    vq = oracle.quant_v(v, p)
    t_quant = time.perf_counter() - t0
    nqb = qk["n_pad"] // 128
    picks = sorted(set(int(x) for x in np.linspace(0, nqb - 1, sample_blocks)))
    t0 = time.perf_counter()
    for qb in picks:
        oracle.emulate_block(qk, vq, 0, 0, qb, w.causal)
    t_blocks = time.perf_counter() - t0
    if w.causal:   # block cost grows with its key count; scale by the mean over blocks
        keys = [min(w.N, 128 * (qb + 1)) for qb in picks]
        mean_keys = sum(min(w.N, 128 * (b + 1)) for b in range(nqb)) / nqb
        per_block = t_blocks / sum(keys) * mean_keys
    else:
        per_block = t_blocks / len(picks)
    t_total = w.B * w.H * (t_quant + nqb * per_block)
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max(blas) if blas else threads
    except Exception:
        pass
    return {"value": w.ops / t_total / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": (f"one head of {w.name}: oracle quantisation of Q,K,V ({t_quant:.2f}s) + tiled emulation of "
                       f"query blocks {picks} ({t_blocks:.2f}s), extrapolated to B*H heads x {nqb} blocks"),
            "seconds_measured": round(t_quant + t_blocks, 2), "seconds_extrapolated": round(t_total, 1)}


def probe_bench(args, w, qt, kt, vt, shape, ws, dev):
    """Time sage_probe_qk_bits (it synchronises the stream itself) on the middle
    query block.  The exact reference is the probe's fp32 vector-ALU part:
    4 * B * H * rows * keys * d flops (QK dot products and the P V sums)."""
    import torch
    from quantized_attention_sage_amd import api
    params = api.make_params(qk_bits=4, gran=w.gran, qk_format="int_e2m3")
    scratch = api.ProbeScratch(shape, dev)
    qb = (w.N - 1) // 128 // 2
    for _ in range(args.warmup):
        api.probe_qk_bits(qt, kt, vt, params, ws, shape, w.causal, qb, args.cos_min, scratch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = api.probe_qk_bits(qt, kt, vt, params, ws, shape, w.causal, qb, args.cos_min, scratch)
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    rows = min(128, w.N - 128 * qb)
    keys = min(w.N, 128 * qb + 128) if w.causal else w.N
    ref_flops = 4 * w.B * w.H * rows * keys * w.d
    print(json.dumps({"metric": "adaptive INT4/INT8 probe time (sage_probe_qk_bits, host-synchronised)",
                      "value": round(ms, 4), "unit": "ms", "higher_is_better": False, "steps": args.steps,
                      "warmup": args.warmup, "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N,
                                                         "d": w.d, "causal": w.causal, "q_block": qb,
                                                         "cos_min": args.cos_min},
                      "reference_flops": ref_flops, "result": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="target")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--qk", choices=("int", "int_e4m3", "int_e2m3", "mxfp4"), default="int",
                    help="Q/K codes: int (INT8 / INT4-range per the workload, the default), int_e4m3 / "
                         "int_e2m3 (the INT4-range codes held as E4M3 bytes / packed FP6 E2M3 on the FP8 / FP6 "
                         "matrix cores; INT4-range workloads only) or mxfp4 (FP4 E2M1 with an E8M0 scale per "
                         "32 channels)")
    ap.add_argument("--pv", choices=("fp8", "f16"), default="fp8",
                    help="P~V precision: fp8 (SageAttention2, the default) or f16 (16-bit P~ and V, "
                         "the first SageAttention's setting)")
    ap.add_argument("--probe", action="store_true",
                    help="time the adaptive INT4/INT8 probe (sage_probe_qk_bits on the middle query block) "
                         "instead of the step, and print its own JSON line")
    ap.add_argument("--cos-min", type=float, default=0.999, help="cosine-similarity bar of --probe")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run 3 plain 1 GiB device-to-device elementwise copies (neg) whose "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the HBM traffic figure")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here "
              "(heads would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from quantized_attention_sage_amd import api
    from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, describe

    w = WORKLOADS[args.workload]
    if args.qk in ("int_e4m3", "int_e2m3") and w.qk_bits != 4:
        print(f"--qk {args.qk} holds INT4-range codes; workload {w.name} uses INT{w.qk_bits}", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    q, k, v = make_inputs(w)
    qt, kt, vt = (torch.from_numpy(x).to(tdt).to(dev) for x in (q, k, v))
    del q, k, v
    params = api.make_params(qk_bits=w.qk_bits, gran=w.gran, pv=args.pv, qk_format=args.qk)
    shape = api.make_shape(qt, kt, vt)
    ws = api.Workspace(shape, params, dev)
    out = torch.empty_like(qt)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        api.quant_qk(qt, kt, vt, params, ws, shape)
        if ev is not None:
            ev[1].record(stream)
        api.quant_v(vt, params, ws, shape)
        if ev is not None:
            ev[2].record(stream)
        api.attn_fwd(ws, shape, params, w.causal, out)
        if ev is not None:
            ev[3].record(stream)

    if args.probe:
        if args.qk == "mxfp4" or args.pv != "fp8":
            print("--probe compares integer Q/K codes with FP8 P~V: leave --qk and --pv at their defaults",
                  file=sys.stderr)
            sys.exit(2)
        probe_bench(args, w, qt, kt, vt, shape, ws, dev)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # Per-kernel-group durations with HIP events on the launch stream (separate pass).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    qk_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    v_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    tops = w.ops / (ms_per_step * 1e-3) / 1e12
    attn_tops = w.ops / (attn_ms * 1e-3) / 1e12
    pv16, mx = args.pv == "f16", args.qk == "mxfp4"
    # FP4 and FP6 share the 10.1 P/s dense rate: the E2M3-held codes are priced like MXFP4 (QK at that rate,
    # P~V at the FP8 rate, half the operations each)
    peak = PEAK_PV16_TOPS if pv16 else (PEAK_MXFP4_TOPS if (mx or args.qk == "int_e2m3") else PEAK_TOPS)
    traffic = None if (pv16 or mx or args.qk != "int") else traffic_from_profile(w.name)
    qk_bytes, v_bytes = quant_bytes(w, args.pv, args.qk)
    rec = {
        "metric": "attention TOPS (4*B*H*N^2*d, halved if causal) of quant_qk + quant_v + attn_fwd",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (("mxfp4 QK" if mx else ("int8 QK" if w.qk_bits == 8 else
                                          ("int4-range QK as " + args.qk[4:] if args.qk != "int" else "int4-range QK"))) +
                  (f" / {w.dtype} PV" if pv16 else " / fp8 PV") + f" ({w.dtype} in/out)"),
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "io_dtype": w.dtype, "qk": "mxfp4" if mx else f"int{w.qk_bits}" + (args.qk[3:] if args.qk != "int" else ""),
                   "granularity": w.gran,
                   "pv": args.pv},
        "roofline": {"bound": "mfma", "achieved": round(attn_tops, 1), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(attn_tops / peak, 4), "traffic": traffic,
                     "kernel": "attn_pvh_kernel" if pv16 else ("attn_fp4_kernel" if mx else "attn_fwd_kernel"),
                     "kernel_ms": round(attn_ms, 4),
                     "ops_per_launch": w.ops},
        "breakdown_ms": {"quant_qk": round(qk_ms, 4), "quant_v": round(v_ms, 4), "attn_fwd": round(attn_ms, 4)},
        "quant_roofline": {
            "bound": "hbm", "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "quant_qk": {"bytes": qk_bytes, "achieved": round(qk_bytes / (qk_ms * 1e6), 1),
                         "frac": round(qk_bytes / (qk_ms * 1e6) / PEAK_HBM_GBPS, 4)},
            "quant_v": {"bytes": v_bytes, "achieved": round(v_bytes / (v_ms * 1e6), 1),
                        "frac": round(v_bytes / (v_ms * 1e6) / PEAK_HBM_GBPS, 4)},
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, pv=args.pv, qk_format=args.qk)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
