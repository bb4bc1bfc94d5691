#!/usr/bin/env python3
"""Throughput of the quantized attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload target] [--gpus 1]

One step = sage_quant_qk + sage_quant_v + sage_attn_fwd over one batch of
synthetic inputs already resident in HBM.  Prints ONE JSON line.  `value` is
attention TOPS of the whole step: 4*B*H*N^2*d (halved when causal) divided by
the step time.  `roofline` covers the attention kernel, timed with HIP events
on the stream it is launched on.  `cpu_baseline` times the CPU oracle
(quantisation emulation plus tiled attention emulation, and exact fp64
attention) on a bounded sample of the same workload and extrapolates it;
`accuracy` compares the GPU output with both on those sampled rows.
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


QUANT_COUNTERS = os.path.join(ROOT, "profiles", "quant_counters.json")


def quant_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("quant.hip", "sage_internal.h"):
        with open(os.path.join(ROOT, "quantized_attention_sage_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def quant_traffic_from_profile(workload: str):
    """HBM bytes per call of the two quantisation calls ({"quant_qk": B, "quant_v": B})
    from the committed rocprofv3 counter summary, or None when it is missing or
    the kernels changed since."""
    try:
        with open(QUANT_COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != quant_source_hash() or rec.get("workload") != workload:
        return None
    return {c: v["hbm_bytes"] for c, v in rec.get("calls", {}).items()}


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


NOMINAL_GHZ = 2.4   # the clock the published matrix peaks are quoted at
N_XCD = 8


def cycles_from_profile(workload: str):
    """GPU cycles per attention launch on one XCD (GRBM_GUI_ACTIVE summed over
    the 8 XCDs, divided by 8) from the committed rocprofv3 counter summary, or
    None when it is missing or the kernel changed since."""
    try:
        with open(COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    g = rec.get("grbm_gui_active_per_dispatch")
    return None if g is None else g / N_XCD


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _emulate_head(job):
    """One worker of the emulation timing: the oracle's quantisation of one head
    plus the tiled emulation of the given query blocks (one BLAS thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle.quant import QuantParams
    q, k, v, params, blocks, causal = job
    with threadpool_limits(1):
        p = QuantParams(**params)
        t0 = time.perf_counter()
        qk = oracle.quant_qk(q, k, p, with_bias=False)
        vq = oracle.quant_v(v, p)
        t_quant = time.perf_counter() - t0
        outs = []
        t0 = time.perf_counter()
        for qb in blocks:
            o, rows = oracle.emulate_block(qk, vq, 0, 0, qb, causal)
            outs.append(o)
        t_blocks = time.perf_counter() - t0
    return t_quant, t_blocks, np.concatenate(outs)


def cpu_baseline(w, q, k, v, out_gpu, pv: str = "fp8", qk_format: str = "int", blocks_per_head: int = 12):
    """Time the oracle (as it stands) on a bounded sample of the workload, on the
    host's cores, and compare the GPU output with it on the same rows.

    Sample: P heads spread over B*H (P = worker processes, at most 16) and
    `blocks_per_head` query blocks spread over each head's blocks.
      * emulation (the quantised method): one process per head, each running
        the oracle's quantisation of its head and the tiled emulation of its
        blocks; extrapolated to B*H heads x all blocks at P heads in parallel;
      * exact fp64 attention of the same rows through BLAS on all P cores,
        extrapolated the same way.
    The GPU output of those rows is then checked against both (the accuracy of
    the measured line: cosine similarity and relative L1 against exact
    attention, the metrics of the SageAttention2++ summary's "A.2 Datasets and
    Metrics"; max |O - emulation| against the 2e-3 max|V| bar)."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    nqb = -(-w.N // 128)
    heads = sorted(set(int(x) for x in np.linspace(0, w.B * w.H - 1, min(cores, w.B * w.H))))
    picks = sorted(set(int(x) for x in np.linspace(0, nqb - 1, min(blocks_per_head, nqb))))
    params = dict(qk_bits=w.qk_bits, gran=w.gran, pv=w.dtype if pv == "f16" else "fp8", qk_format=qk_format)
    jobs = []
    for bh in heads:
        b, h = divmod(bh, w.H)
        jobs.append((q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], params, picks, w.causal))
    ctx = mp.get_context("spawn")   # workers touch no GPU state and start from a clean interpreter
    t0 = time.perf_counter()
    with ctx.Pool(len(jobs)) as pool:
        res = pool.map(_emulate_head, jobs)
    wall_emul = time.perf_counter() - t0

    keys = [min(w.N, 128 * (qb + 1)) if w.causal else w.N for qb in picks]
    mean_keys = (sum(min(w.N, 128 * (b + 1)) for b in range(nqb)) / nqb) if w.causal else w.N
    # per head: quantisation + every block at the sampled per-key cost; heads run P at a time
    per_head = [tq + tb / sum(keys) * mean_keys * nqb for (tq, tb, _) in res]
    t_emul = float(np.mean(per_head)) * (w.B * w.H) / len(jobs)

    rows = np.concatenate([np.arange(128 * qb, min(w.N, 128 * qb + 128)) for qb in picks])
    ex_rows = []
    t0 = time.perf_counter()
    with threadpool_limits(cores):
        for bh in heads:
            b, h = divmod(bh, w.H)
            ex_rows.append(oracle.exact_attention_rows(q[b, h], k[b, h], v[b, h], rows, w.causal))
    t_exact_s = time.perf_counter() - t0
    # exact attention costs the same for every row (all N keys, masked when causal)
    t_exact = t_exact_s * (w.B * w.H * w.N) / (len(heads) * len(rows))

    gpu = np.concatenate([out_gpu[divmod(bh, w.H)][rows] for bh in heads]).astype(np.float64)
    ex = np.concatenate(ex_rows)
    em = np.concatenate([r[2] for r in res])
    cos = float((gpu.ravel() @ ex.ravel()) / (np.linalg.norm(gpu) * np.linalg.norm(ex)))
    rl1 = float(np.abs(gpu - ex).sum() / np.abs(ex).sum())
    cos_e = float((em.ravel() @ ex.ravel()) / (np.linalg.norm(em) * np.linalg.norm(ex)))
    rl1_e = float(np.abs(em - ex).sum() / np.abs(ex).sum())
    tol = 2e-3 * float(np.abs(v).max())
    accuracy = {
        "rows": f"query blocks {picks} of heads {heads} ({len(rows) * len(heads)} rows)",
        "vs_exact": {"cos": round(cos, 6), "rel_l1": round(rl1, 5),
                     "bar": {"cos": 0.999, "rel_l1": 0.02}, "met": bool(cos >= 0.999 and rl1 <= 0.02)},
        "emulation_vs_exact": {"cos": round(cos_e, 6), "rel_l1": round(rl1_e, 5)},
        "vs_emulation": {"max_abs_err": float(np.abs(gpu - em).max()), "tol": tol,
                         "frac_of_tol": round(float(np.abs(gpu - em).max()) / tol, 4)},
    }
    base = {"value": w.ops / t_emul / 1e12, "unit": "TOPS", "cores": len(jobs), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": (f"{w.name}: heads {heads} (one process each, one BLAS thread) x query blocks {picks}: "
                       f"oracle quantisation of the head + tiled emulation of the blocks "
                       f"({wall_emul:.1f}s wall), extrapolated to {w.B * w.H} heads x {nqb} blocks"),
            "seconds_measured": round(wall_emul, 2), "seconds_extrapolated": round(t_emul, 1),
            "exact_fp64": {"value": w.ops / t_exact / 1e12, "unit": "TOPS", "cores": cores,
                           "sample": f"exact fp64 attention of the same {len(rows) * len(heads)} rows through BLAS "
                                     f"({t_exact_s:.1f}s), extrapolated to the workload",
                           "seconds_measured": round(t_exact_s, 2), "seconds_extrapolated": round(t_exact, 1)}}
    return base, accuracy


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


def backward_bench(args, w, qt, kt, vt, params, shape, ws, out, dev):
    """One 8-bit training step: sage_quant_qk + sage_quant_v + sage_attn_fwd_lse
    + sage_attn_bwd, timed whole and by part (HIP events on the launch stream).
    Backward operations: the five products of the FlashAttention backward,
    10 * B * H * N^2 * d (halved when causal); the forward's 4 * B * H * N^2 * d."""
    import numpy as np
    import torch
    from quantized_attention_sage_amd import api
    from quantized_attention_sage_amd.workloads import make_grad
    do = torch.from_numpy(make_grad(w)).to(qt.dtype).to(dev)
    lse = torch.empty((w.B, w.H, ws.layout.n_pad), dtype=torch.float32, device=dev)
    bws = api.BwdWorkspace(shape, params, dev)
    grads = [torch.empty(qt.shape, dtype=torch.float32, device=dev) for _ in range(3)]
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        api.quant_qk(qt, kt, vt, params, ws, shape)
        api.quant_v(vt, params, ws, shape)
        api.attn_fwd_lse(ws, shape, params, w.causal, out, lse)
        if ev is not None:
            ev[1].record(stream)
        api.attn_bwd(qt, kt, vt, out, do, lse, ws, shape, params, w.causal, bws, *grads)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    bwd_ops = w.ops * 2.5
    print(json.dumps({
        "metric": "8-bit attention training step TOPS ((4 + 10) * B*H*N^2*d, halved if causal) of "
                  "quant_qk + quant_v + attn_fwd_lse + attn_bwd",
        "value": round((w.ops + bwd_ops) / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": "int8 QK, dP / fp8 PV, dV, dQ, dK (" + w.dtype + " in, fp32 gradients)", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal},
        "breakdown_ms": {"forward": round(fwd_ms, 4), "backward": round(bwd_ms, 4)},
        "backward_roofline": {"bound": "mfma", "achieved": round(bwd_ops / (bwd_ms * 1e-3) / 1e12, 1),
                              "peak": PEAK_TOPS, "unit": "TFLOP/s",
                              "frac": round(bwd_ops / (bwd_ms * 1e-3) / 1e12 / PEAK_TOPS, 4),
                              "ops_per_call": bwd_ops},
    }), flush=True)


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
    ap.add_argument("--backward", action="store_true",
                    help="time one 8-bit training step (forward with its row log-sum-exp plus the backward) "
                         "instead of the inference step, and print its own JSON line")
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

    if args.backward:
        if args.qk != "int" or args.pv != "fp8" or w.qk_bits != 8 or w.gran != "thread":
            print("--backward runs INT8 Q/K codes (THREAD groups) with FP8 P~V", file=sys.stderr)
            sys.exit(2)
        backward_bench(args, w, qt, kt, vt, params, shape, ws, out, dev)
        return

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
    attn_ms_median = float(np.median([e[2].elapsed_time(e[3]) for e in evs]))

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
    qtraffic = None if (pv16 or mx or args.qk != "int") else quant_traffic_from_profile(w.name)
    qk_bytes, v_bytes = quant_bytes(w, args.pv, args.qk)
    # The clock the kernel sustains: its cycles per launch (a count of work,
    # much the same on every box) over this run's launch time.
    cycles = None if (pv16 or mx or args.qk != "int") else cycles_from_profile(w.name)
    clock = None
    if cycles is not None:
        ghz = cycles / (attn_ms * 1e-3) / 1e9
        clock = {"ghz": round(ghz, 3), "cycles_per_launch": round(cycles),
                 "frac_at_clock": round(attn_tops / (peak * ghz / NOMINAL_GHZ), 4),
                 "source": "GRBM_GUI_ACTIVE per XCD per launch (profiles/attn_fwd_counters.json) "
                           "over this run's launch time"}
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
                     "kernel_ms": round(attn_ms, 4), "kernel_ms_median": round(attn_ms_median, 4),
                     "ops_per_launch": w.ops, "sustained_clock": clock},
        "breakdown_ms": {"quant_qk": round(qk_ms, 4), "quant_v": round(v_ms, 4), "attn_fwd": round(attn_ms, 4)},
        "quant_roofline": {
            "bound": "hbm", "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "quant_qk": {"bytes": qk_bytes, "achieved": round(qk_bytes / (qk_ms * 1e6), 1),
                         "frac": round(qk_bytes / (qk_ms * 1e6) / PEAK_HBM_GBPS, 4),
                         "traffic": (qtraffic or {}).get("quant_qk")},
            "quant_v": {"bytes": v_bytes, "achieved": round(v_bytes / (v_ms * 1e6), 1),
                        "frac": round(v_bytes / (v_ms * 1e6) / PEAK_HBM_GBPS, 4),
                        "traffic": (qtraffic or {}).get("quant_v")},
        },
    }
    rec["accuracy"] = None
    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()
        rec["cpu_baseline"], rec["accuracy"] = cpu_baseline(w, q, k, v, out.float().cpu().numpy(), pv=args.pv,
                                                            qk_format=args.qk)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
