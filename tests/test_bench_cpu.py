"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic work
each call is credited with and its roofline class, the rate helpers, and the
rule that recorded HBM traffic is reported only for unchanged kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_layer_counts_prefill_7b():
    M, N, K = 8192, 4096, 4096
    c = bench.layer_counts(M, N, K, 2, 2, gy=False)
    assert c["act_quant"]["bytes"] == M * K * 2 + M * K + 4 * M
    assert c["weight_quant"]["bytes"] == 2 * N * K * 2 + N * K // 4 + 4
    assert c["quant_operands"]["bytes"] == c["act_quant"]["bytes"] + c["weight_quant"]["bytes"]
    assert c["linear_fwd"]["ops"] == 2 * M * N * K
    assert c["linear_fwd"]["bytes"] == M * K + N * K // 4 + 4 * M + 4 * M * N
    # arithmetic intensity ~1600 op/B, above the int8 ridge (5000 TOPS / 8 TB/s = 625)
    assert c["linear_fwd"]["bound"] == "mfma"
    assert c["act_quant"]["bound"] == "hbm" and "linear_bwd_ste" not in c


def test_layer_counts_small_llama_training():
    M, N, K = 8192, 1376, 512
    c = bench.layer_counts(M, N, K, 2, 4, gy=True)
    # the forward's fp32 y write makes the small layer HBM-bound (AI ~ 233 < 625)
    assert c["linear_fwd"]["bound"] == "hbm"
    assert c["bwd_grad_x"]["ops"] == c["bwd_grad_W"]["ops"] == 2 * M * N * K
    assert c["linear_bwd_ste"]["ops"] == 4 * M * N * K
    assert c["bwd_grad_W"]["bytes"] == 2 * M * N + M * K + 4 * M + 4 * N * K
    assert c["weight_quant_counted"]["bytes"] == c["weight_quant"]["bytes"] + 32


def test_rate_helpers():
    e = bench.hbm_entry(0.5, 4 * 10**9, ceiling_gbs=5000.0)
    assert e["achieved"] == pytest.approx(8000.0) and e["frac"] == pytest.approx(1.0)
    assert e["frac_of_ceiling"] == pytest.approx(1.6)
    m = bench.mfma_entry(0.1, 250 * 10**12 // 1000, bench.INT8_PEAK_TOPS)
    assert m["achieved"] == pytest.approx(2500.0) and m["frac"] == pytest.approx(0.5)


def test_traffic_is_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    rec = {"fetch_bytes": 100, "write_bytes": 20, "kernels": ["k"]}
    good = dict(rec, source_sha256=bench.source_digest("linear_fwd"))
    stale = dict(rec, source_sha256="0" * 64)
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"linear_fwd@prefill_7b": good, "weight_quant@prefill_7b": stale}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("linear_fwd", "prefill_7b") == 120
    assert bench.measured_traffic("weight_quant", "prefill_7b") is None
    assert bench.measured_traffic("act_quant", "prefill_7b") is None


def test_every_recorded_call_has_its_sources_listed():
    # a call without a source list hashes common.h alone and its recorded
    # traffic could never be reported
    with open(bench.TRAFFIC_FILE) as f:
        recs = json.load(f)
    for key in recs:
        call = key.split("@")[0]
        assert bench.SOURCES_OF.get(call), f"{key}: no kernel sources listed for {call}"
