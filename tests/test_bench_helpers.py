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
