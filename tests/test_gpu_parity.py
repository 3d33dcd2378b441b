"""GPU parity of the HIP kernels (through the C ABI) against the CPU oracle.

Full tensors at sizes the oracle finishes in seconds (several query tiles and
key blocks, ragged tails, GQA, both head-dim shapes, edge sizes), bit-exact
special cases, run-to-run determinism, and the full-size workloads in the launch
configuration the benchmark times, compared on sampled rows.
"""
import hashlib

import numpy as np
import pytest
import torch

from parity import (W, binding, check_fp8, gpu_select, oracle_bf16, oracle_fp8, rel_rms, row_rel_rms,
                    row0_expected_fp8, run_bf16, run_fp8, NORTH_STAR_FP8, TOL_BF16, TOL_BF16_ROW)
from oracle.e4m3 import bf16_rne, decode_e4m3

pytestmark = pytest.mark.gpu
MODES = ["exact", "lean"]


def custom(B, Hq, Hkv, S, dqk, seed=1234):
    return W.Workload(f"custom_B{B}_H{Hq}x{Hkv}_S{S}_d{dqk}", B, Hq, Hkv, S, dqk, 128)


@pytest.mark.parametrize("mode", MODES)
def test_tiny_full_tensor(mode):
    w = W.WORKLOADS["tiny"]
    d = W.make_fp8(w)
    out = run_fp8(d, mode)
    got = gpu_select(out)
    emu, ref = oracle_fp8(d, mode)
    check_fp8(got, emu, ref, f"tiny {mode}", d=d, mode=mode)
    # row 0 has a single visible key: bit-exact
    exp0 = row0_expected_fp8(d)
    assert np.array_equal(got[:, 0].astype(np.float32), exp0), "row 0 not bit-exact"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [
    (1, 2, 2, 1, 128), (1, 2, 1, 2, 128), (1, 2, 2, 63, 128), (1, 2, 2, 64, 128), (1, 2, 2, 65, 128),
    (2, 4, 2, 129, 128), (1, 4, 1, 200, 192), (1, 2, 2, 333, 128), (2, 4, 4, 515, 192),
    (1, 8, 2, 1000, 128), (1, 64, 2, 300, 128), (3, 16, 16, 70, 192), (1, 32, 1, 257, 192),
])
def test_ragged_and_gqa_full_tensor(shape, mode):
    B, Hq, Hkv, S, dqk = shape
    w = custom(B, Hq, Hkv, S, dqk)
    d = W.make_fp8(w, seed=777 + S)
    out = run_fp8(d, mode)
    got = gpu_select(out)
    emu, ref = oracle_fp8(d, mode)
    check_fp8(got, emu, ref, f"{w.name} {mode}", d=d, mode=mode)
    assert np.array_equal(got[:, 0].astype(np.float32), row0_expected_fp8(d)[:, np.arange(Hq) // (Hq // Hkv)])


# More than 32 query heads in all with K/V heads in multiples of 8: the workgroups run in
# bands of tiles of one query head, the heads of one K/V head on one XCD (with GQA, the
# query heads of a K/V head adjacent); every (tile, head) must be computed once.
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(2, 32, 4, 300, 128), (1, 40, 8, 300, 192), (1, 64, 64, 140, 128)])
def test_banded_tile_order_full_tensor(shape, mode):
    B, Hq, Hkv, S, dqk = shape
    w = custom(B, Hq, Hkv, S, dqk)
    d = W.make_fp8(w, seed=901 + S)
    got = gpu_select(run_fp8(d, mode))
    emu, ref = oracle_fp8(d, mode)
    check_fp8(got, emu, ref, f"{w.name} {mode}", d=d, mode=mode)
    assert np.array_equal(got[:, 0].astype(np.float32), row0_expected_fp8(d)[:, np.arange(Hq) // (Hq // Hkv)])


@pytest.mark.parametrize("mode", MODES)
def test_banded_tile_order_full_band_sampled(mode):
    # 33 query tiles per head: one full band of 32 tiles and a partial band of one
    B, Hq, Hkv, S = 2, 32, 8, 32 * 256 + 100
    w = custom(B, Hq, Hkv, S, 128)
    d = W.make_fp8(w, seed=4242)
    out = run_fp8(d, mode)
    rows = np.unique(np.concatenate([np.arange(0, S, 97), np.arange(S - 300, S)]))
    heads = [0, 5, 17, 31]
    got = gpu_select(out, heads=heads, rows=rows)
    assert bool(torch.isfinite(out).all())
    del out
    emu, ref = oracle_fp8(d, mode, heads=heads, rows=rows)
    check_fp8(got, emu, ref, f"{w.name} {mode} (rows={len(rows)}, heads={heads})", rows=rows, d=d, mode=mode,
              heads=heads)


@pytest.mark.parametrize("mode", MODES)
def test_zero_query_is_prefix_mean(mode):
    w = custom(1, 2, 2, 300, 128)
    d = W.make_fp8(w, seed=5)
    d["q8"] = torch.zeros_like(d["q8"])
    got = gpu_select(run_fp8(d, mode))
    vd = decode_e4m3(d["v8"].numpy())
    pm = d["v_scale"] * np.cumsum(vd, axis=1) / np.arange(1, 301)[None, :, None, None]
    # all p~ = 256 -> exact weights; only fp32 accumulation order and bf16 output rounding remain
    assert np.max(np.abs(got - pm) / (np.abs(pm) + 1e-3)) < 2 ** -7


def test_empty_problem_launches_nothing():
    z = torch.zeros((1, 0, 2, 128), dtype=torch.uint8, device="cuda:0")
    out = binding.attn_fwd_fp8(z, z, z, 1.0, 1.0, 1.0)
    assert out.shape == (1, 0, 2, 128)


@pytest.mark.parametrize("mode", MODES)
def test_deterministic_over_repeated_launches(mode):
    w = custom(1, 8, 8, 4096, 128)
    d = W.make_fp8(w, seed=99)
    q8, k8, v8 = (d[n].to("cuda:0") for n in ("q8", "k8", "v8"))
    out = torch.empty((1, 4096, 8, 128), dtype=torch.bfloat16, device="cuda:0")
    first, mismatches = None, 0
    for _ in range(300):
        binding.attn_fwd_fp8(q8, k8, v8, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=mode, out=out)
        if first is None:
            first = out.view(torch.uint8).clone()
        elif not torch.equal(out.view(torch.uint8), first):
            mismatches += 1
    torch.cuda.synchronize()
    assert mismatches == 0
    digests = {hashlib.sha256(first.cpu().numpy().tobytes()).hexdigest(),
               hashlib.sha256(out.view(torch.uint8).cpu().numpy().tobytes()).hexdigest()}
    assert len(digests) == 1


def _sampled_heads(Hq):
    return sorted({0, Hq // 2, Hq - 1})


# Full-size workloads in the launch configuration the benchmark times: 1024 query rows per
# sampled head, 7/8 of them from the second half of the sequence (the long causal rows that
# carry almost all of the work), checked row by row.
FULL_ROWS = 1024
_full_cache = {}


def _full(name, mode):
    key = (name, mode)
    if key not in _full_cache:
        _full_cache.clear()
        w = W.WORKLOADS[name]
        d = W.make_fp8(w)
        out = run_fp8(d, mode)
        rows = W.sample_rows_long(w.S, FULL_ROWS).numpy()
        heads = _sampled_heads(w.Hq)
        got = gpu_select(out, heads=heads, rows=rows)
        finite = bool(torch.isfinite(out).all())
        del out
        emu, ref = oracle_fp8(d, mode, heads=heads, rows=rows)
        _full_cache[key] = (w, d, rows, heads, got, emu, ref, finite)
    return _full_cache[key]


FULL_CASES = [("gauss32k", "exact"), ("gauss32k", "lean"), ("mistral", "exact"), ("mistral", "lean"),
              ("qwen", "exact"), ("qwen", "lean"), ("mla", "exact"), ("mla", "lean")]


@pytest.mark.parametrize("name,mode", FULL_CASES)
def test_full_size_workloads_sampled(name, mode):
    w, d, rows, heads, got, emu, ref, finite = _full(name, mode)
    check_fp8(got, emu, ref, f"{name} {mode} (rows={len(rows)}, heads={heads})", rows=rows, d=d, mode=mode,
              heads=heads)
    assert np.array_equal(got[:, 0].astype(np.float32),
                          row0_expected_fp8(d)[:, np.array(heads) // (w.Hq // w.Hkv)])
    # every output finite, not only the sampled ones
    assert finite


@pytest.mark.parametrize("name,mode", FULL_CASES)
def test_north_star_fixed_fp64_bar(name, mode):
    """The fixed 2e-2 relative-RMS bar against fp64 over the whole output tensor, reported on
    its own.  The whole-tensor figure is estimated from every row below 256 plus a uniform
    sample of 1024 later rows, each weighted by the number of rows it stands for (three heads).

    Rounding every probability to e4m3 leaves a floor of ~2.65% (exact) and ~3.14% (Lean P)
    on each long row of Gaussian-like inputs (closed form in tests/test_oracle_emulate.py), so
    where the method itself - the emulation - is above the bar the GPU cannot meet it either:
    that case is an expected failure, after checking that the GPU is at the method's error."""
    w = W.WORKLOADS[name]
    d = W.make_fp8(w)
    out = run_fp8(d, mode)
    rows, wts = W.sample_rows_strata(w.S)
    rows, wts = rows.numpy(), wts.numpy()
    heads = _sampled_heads(w.Hq)
    got = gpu_select(out, heads=heads, rows=rows)
    del out
    emu, ref = oracle_fp8(d, mode, heads=heads, rows=rows)

    def whole(x):
        num = np.sum(wts[None, :, None] * np.sum((x - ref) ** 2, axis=-1))
        return float(np.sqrt(num / np.sum(wts[None, :, None] * np.sum(ref ** 2, axis=-1))))
    e_gpu, e_emu = whole(got), whole(emu)
    late = rows >= w.S // 2
    e_long = float(np.sqrt(np.mean(row_rel_rms(got[:, late], ref[:, late]) ** 2)))
    print(f"[north-star] {name} {mode}: whole-tensor GPU vs fp64 {e_gpu:.4f} (emulation {e_emu:.4f}); "
          f"rows in the second half, RMS of per-row errors {e_long:.4f}")
    if e_gpu <= NORTH_STAR_FP8:
        return
    assert e_emu > NORTH_STAR_FP8 - 1e-3 and abs(e_gpu - e_emu) < 2e-3, (e_gpu, e_emu)
    pytest.xfail(f"the method's own error against fp64 ({e_emu:.4f}) is above 2e-2; GPU {e_gpu:.4f}")


# ----------------------------------------------------------------------------- BF16

@pytest.mark.parametrize("shape", [(1, 2, 2, 256, 128), (2, 4, 2, 129, 128), (1, 4, 1, 333, 192),
                                   (1, 2, 2, 1, 128), (1, 2, 2, 65, 192),
                                   # more than 32 query heads, K/V heads in multiples of 8: banded order
                                   (2, 32, 4, 300, 128), (1, 40, 8, 300, 192)])
def test_bf16_full_tensor(shape):
    B, Hq, Hkv, S, dqk = shape
    d = W.make_bf16(custom(B, Hq, Hkv, S, dqk), seed=31 + S)
    got = gpu_select(run_bf16(d))
    ref = oracle_bf16(d)
    e = rel_rms(got, ref)
    er = row_rel_rms(got, ref)
    print(f"[parity] bf16 {shape}: vs fp64 {e:.2e}; per row max {er.max():.2e}")
    assert np.all(np.isfinite(got)) and e <= TOL_BF16 and er.max() <= TOL_BF16_ROW
    # row 0: O_0 = v_0 * bf16(p)/p, within one bf16 ulp of v_0
    v0 = d["v"][:, 0].float().numpy()[:, np.arange(Hq) // (Hq // Hkv)]
    assert np.all(np.abs(got[:, 0] - v0) <= 2.0 ** -7 * np.abs(v0) + 1e-30)


@pytest.mark.parametrize("dqk", [128, 192])
def test_bf16_deterministic_over_repeated_launches(dqk):
    w = custom(1, 8, 2, 2048, dqk)
    d = W.make_bf16(w, seed=77)
    q, k, v = (d[n].to("cuda:0") for n in ("q", "k", "v"))
    out = torch.empty((1, 2048, 8, 128), dtype=torch.bfloat16, device="cuda:0")
    first, mismatches = None, 0
    for _ in range(200):
        binding.attn_fwd_bf16(q, k, v, out=out)
        if first is None:
            first = out.view(torch.int16).clone()
        elif not torch.equal(out.view(torch.int16), first):
            mismatches += 1
    torch.cuda.synchronize()
    assert mismatches == 0


@pytest.mark.parametrize("name", ["qwen", "mla"])
def test_bf16_full_size_sampled(name):
    w = W.WORKLOADS[name]
    d = W.make_bf16(w)
    out = run_bf16(d)
    rows = W.sample_rows_long(w.S, FULL_ROWS).numpy()
    heads = _sampled_heads(w.Hq)
    got = gpu_select(out, heads=heads, rows=rows)
    ref = oracle_bf16(d, heads=heads, rows=rows)
    e = rel_rms(got, ref)
    er = row_rel_rms(got, ref)
    print(f"[parity] bf16 {name}: vs fp64 {e:.2e}; per row median {np.median(er):.2e} max {er.max():.2e}")
    assert e <= TOL_BF16 and bool(torch.isfinite(out).all())
    assert er.max() <= TOL_BF16_ROW
