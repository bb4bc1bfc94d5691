"""Host-side logic of bench.py: the algorithmic byte model of the two
quantisation calls, the committed counter records it reads, and the refusal
of more than one GPU.  No GPU needed."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quantized_attention_sage_amd.workloads import WORKLOADS  # noqa: E402


def test_quant_bytes_by_hand():
    # B=1, H=32, N=16384, d=128: 2^24 positions per tensor, 128 query blocks
    w = WORKLOADS["target"]
    pos = 32 * 16384 * 128
    qk, v = bench.quant_bytes(w)
    assert qk == 2 * 2 * pos + 2 * pos + 32 * 128 * 16384 * 4
    assert v == 2 * pos + pos
    _, v16 = bench.quant_bytes(w, pv="f16")
    assert v16 == 4 * pos
    qk4, _ = bench.quant_bytes(w, qk_format="mxfp4")
    assert qk4 == 4 * pos + 2 * (pos // 2 + pos // 32) + 32 * 128 * 16384 * 4


def test_quant_bytes_pads_to_whole_blocks():
    class W:
        B, H, N, d = 1, 2, 130, 64
    qk, v = bench.quant_bytes(W)
    pos, pad = 2 * 130 * 64, 2 * 256 * 64
    assert qk == 4 * pos + 2 * pad + 2 * 2 * 256 * 4
    assert v == 2 * pos + pad


def _load(name):
    with open(os.path.join(ROOT, "profiles", name)) as fh:
        return json.load(fh)


def test_attention_counter_record_is_consistent():
    r = _load("attn_fwd_counters.json")
    assert r["bytes_per_fetch_unit"] == pytest.approx(r["copy_bytes"] / r["copy_fetch_size"])
    assert r["bytes_per_write_unit"] == pytest.approx(r["copy_bytes"] / r["copy_write_size"])
    assert r["hbm_read_bytes_per_launch"] == pytest.approx(r["fetch_size_per_dispatch"] * r["bytes_per_fetch_unit"])
    assert r["hbm_bytes_per_launch"] == pytest.approx(r["hbm_read_bytes_per_launch"] + r["hbm_write_bytes_per_launch"])
    # the output is written once: bf16 O of the workload
    w = WORKLOADS[r["workload"]]
    assert r["hbm_write_bytes_per_launch"] == pytest.approx(2 * w.B * w.H * w.N * w.d, rel=0.01)


def test_quant_counter_record_sums_its_kernels():
    r = _load("quant_counters.json")
    calls = {"quant_qk": ("q_quant_k_sums_kernel", "k_mean_kernel", "k_quant_bias_kernel"),
             "quant_v": ("v_stats_kernel", "v_finalize_kernel", "v_encode_kernel")}
    w = WORKLOADS[r["workload"]]
    for call, ks in calls.items():
        c = r["calls"][call]
        assert c["hbm_read_bytes"] == pytest.approx(sum(r["kernels"][k]["hbm_read_bytes"] for k in ks))
        assert c["hbm_write_bytes"] == pytest.approx(sum(r["kernels"][k]["hbm_write_bytes"] for k in ks))
        assert c["hbm_bytes"] == pytest.approx(c["hbm_read_bytes"] + c["hbm_write_bytes"])
    # every call reads its inputs at least once and writes at least its codes
    qk, v = bench.quant_bytes(w)
    assert r["calls"]["quant_qk"]["hbm_bytes"] >= 0.99 * qk
    assert r["calls"]["quant_v"]["hbm_bytes"] >= 0.99 * v


def test_counter_records_follow_the_sources(tmp_path, monkeypatch):
    r = _load("quant_counters.json")
    got = bench.quant_traffic_from_profile(r["workload"])
    if r["kernel_source_hash"] == bench.quant_source_hash():
        assert got == {c: v["hbm_bytes"] for c, v in r["calls"].items()}
    else:
        assert got is None
    assert bench.quant_traffic_from_profile("no such workload") is None
    stale = dict(r, kernel_source_hash="0" * 16)
    p = tmp_path / "q.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "QUANT_COUNTERS", str(p))
    assert bench.quant_traffic_from_profile(r["workload"]) is None
    monkeypatch.setattr(bench, "QUANT_COUNTERS", str(tmp_path / "missing.json"))
    assert bench.quant_traffic_from_profile(r["workload"]) is None


def test_clock_record_is_consistent(tmp_path, monkeypatch):
    r = _load("attn_fwd_counters.json")
    # GRBM_GUI_ACTIVE is summed over the 8 XCDs; its per-XCD count over the
    # dispatch time under counters is the clock in that run
    assert r["clock_ghz_under_counters"] == pytest.approx(r["grbm_gui_active_per_dispatch"] / 8
                                                          / (r["dispatch_us_under_counters"] * 1e3))
    assert 1.0 < r["clock_ghz_under_counters"] <= 2.4
    got = bench.cycles_from_profile(r["workload"])
    if r["kernel_source_hash"] == bench.kernel_source_hash():
        assert got == pytest.approx(r["grbm_gui_active_per_dispatch"] / 8)
    else:
        assert got is None
    p = tmp_path / "a.json"
    p.write_text(json.dumps(dict(r, kernel_source_hash="0" * 16)))
    monkeypatch.setattr(bench, "COUNTERS", str(p))
    assert bench.cycles_from_profile(r["workload"]) is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
