"""Host-side checks of bench.py helpers (no GPU)."""
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_sparse_codes_large_tensor_quantile_and_bounds():
    # more elements than float32 counts exactly (2^24): the sample must stay inside the tensor
    n = (1 << 25) + 3
    g = torch.Generator().manual_seed(1)
    x = torch.randint(0, 256, (n,), generator=g, dtype=torch.uint8)
    y = bench.sparse_codes(x)
    zero = y == 0
    assert 0.85 < zero.float().mean().item() < 0.95
    kept = ~zero
    assert torch.equal(y[kept], x[kept])              # kept codes unchanged
    assert int((x[zero] & 0x7F).max()) <= int((x[kept] & 0x7F).min())


def test_sampler_without_sysfs_reports_none():
    s = bench.PowerClockSampler.__new__(bench.PowerClockSampler)
    s.power, s.clock, s.power_file, s.clock_file, s.dpm_file, s.power_cap_w = [], [], None, None, None, None
    r = s.summary(1e12, 1.0)
    assert r["power_w_avg"] is None and r["tflop_per_joule"] is None


def test_cpu_baseline_reports_both_paths_errors_on_a_small_workload():
    import numpy as np
    from fp8_causal_prefill_tiled_amd import workloads as W
    from oracle.attention64 import attention_fp64, dequantize
    w = W.WORKLOADS["tiny"]
    d = W.make_fp8(w)
    ref = attention_fp64(*(dequantize(d[n + "8"].numpy(), d[n + "_scale"]) for n in ("q", "k", "v")))
    rng = np.random.default_rng(0)
    outs = {"lean": ref * (1 + 0.01 * rng.standard_normal(ref.shape)), "exact": ref.copy()}
    r = bench.cpu_baseline(w, d, outs, 0.05, "fp8")
    e = r["gpu_error_on_sample"]
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert 0.005 < e["lean"]["rel_rms_vs_fp64_dequantised_inputs"] < 0.02
    assert e["exact"]["rel_rms_vs_fp64_dequantised_inputs"] < 1e-12   # same rows, chunked differently
    # against the unquantised draws the error includes the e4m3 input rounding
    assert e["exact"]["rel_rms_vs_fp64_unquantised_inputs"] > 0.005
    assert r["gpu_rel_rms_vs_oracle_on_sample"] == e["lean"]["rel_rms_vs_fp64_dequantised_inputs"]


def test_e4m3_floor_values():
    # the benchmark's closed-form floor equals the one the oracle's emulation is pinned to
    import bench
    assert abs(bench._e4m3_floor("exact") - 0.0265) < 2e-4
    assert abs(bench._e4m3_floor("lean") - 0.0314) < 2e-4


def test_committed_counters_follow_the_kernel_source(tmp_path, monkeypatch):
    # the counter record is used only while the kernel source it was taken on is unchanged
    import hashlib
    import json
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel v1")
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"source": "k.hip", "source_sha256_16": hashlib.sha256(b"kernel v1").hexdigest()[:16],
           "workload": "gauss32k", "p_mode": "lean", "hbm_read_bytes_per_launch": 10,
           "hbm_write_bytes_per_launch": 5, "valu_per_score": 3.4, "valu_cycles_frac": 0.5,
           "mfma_busy_frac": 0.7, "summary": "profiles/x.md"}
    (prof / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gauss32k", "lean") == 15
    assert bench.valu_roofline("gauss32k", "lean")["valu_instructions_per_score"] == 3.4
    assert bench.measured_traffic("gauss32k", "exact") is None
    src.write_bytes(b"kernel v2")
    assert bench.measured_traffic("gauss32k", "lean") is None
    assert bench.valu_roofline("gauss32k", "lean") is None
    # a record over several files (kernel source, headers, build flags) follows each of them
    hdr = tmp_path / "k.h"
    hdr.write_bytes(b"header v1")
    rec["sources"] = ["k.hip", "k.h"]
    rec["source_sha256_16"] = hashlib.sha256(b"kernel v2" + b"header v1").hexdigest()[:16]
    (prof / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("gauss32k", "lean") == 15
    hdr.write_bytes(b"header v2")
    assert bench.measured_traffic("gauss32k", "lean") is None
