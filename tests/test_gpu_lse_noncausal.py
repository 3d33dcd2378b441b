"""GPU parity of the non-causal mode (causal=0) and of the per-row log-sum-exp
output (attn_fwd_fp8_lse / attn_fwd_bf16_lse), through the C ABI, against the CPU
oracle on the same seeded inputs.

Bars (derived from the arithmetic):

* O: the same as for the causal path (GPU vs emulation <= 5e-3 relative RMS, vs
  fp64 the method's own error plus output rounding; BF16 <= 4e-3 vs fp64).
* FP8 lse vs the emulation's log of the same rounded-probability denominator:
  fp32 scores and sums leave ~1e-6, so every row is within 2e-4 unless a
  probability whose rounding is ambiguous at the FP8 dot product's precision
  took its other code; such a row must stay within the bound that all of its
  ambiguous probabilities together allow (tests/parity.py, check_lse_fp8).
* FP8 lse vs the fp64 log-sum-exp: the emulation's own bounds (each rounded
  probability within [lo, hi] of its true value when normal, 2^-7 for the
  subnormal rest), plus 1e-3.
* BF16 lse vs fp64 on the bf16 inputs: fp32 scores, exponentials and sums only,
  <= 2e-4 absolute.
"""
import numpy as np
import pytest
import torch

from parity import (W, binding, check_fp8, check_lse_fp8, gpu_select, lse_select, oracle_bf16, oracle_fp8, rel_rms,
                    row_rel_rms, run_bf16, run_fp8, TOL_BF16, TOL_BF16_ROW, TOL_LSE_BF16)
from oracle.e4m3 import decode_e4m3

pytestmark = pytest.mark.gpu
MODES = ["exact", "lean"]


def custom(B, Hq, Hkv, S, dqk):
    return W.Workload(f"custom_B{B}_H{Hq}x{Hkv}_S{S}_d{dqk}", B, Hq, Hkv, S, dqk, 128)


SHAPES = [(1, 2, 2, 1, 128), (1, 2, 2, 65, 128), (2, 4, 2, 129, 128), (1, 4, 1, 200, 192), (1, 2, 2, 333, 128),
          (2, 4, 4, 515, 192), (1, 8, 2, 1000, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", SHAPES)
def test_fp8_output_and_lse_full_tensor(shape, mode, causal):
    B, Hq, Hkv, S, dqk = shape
    w = custom(B, Hq, Hkv, S, dqk)
    d = W.make_fp8(w, seed=4242 + S)
    out, lse = run_fp8(d, mode, causal=causal, return_lse=True)
    emu, ref, lemu, lref = oracle_fp8(d, mode, causal=causal, with_lse=True)
    label = f"{w.name} {mode} causal={causal}"
    check_fp8(gpu_select(out), emu, ref, label, d=d, mode=mode, causal=causal)
    check_lse_fp8(lse_select(lse), lemu, lref, mode, label, d=d, causal=causal)


@pytest.mark.parametrize("mode", MODES)
def test_fp8_lse_does_not_change_the_output(mode):
    # the lse entry point runs the same kernel: O is byte-identical with and without it
    d = W.make_fp8(custom(1, 4, 2, 700, 128), seed=3)
    for causal in (True, False):
        a = run_fp8(d, mode, causal=causal)
        b, _ = run_fp8(d, mode, causal=causal, return_lse=True)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dqk", [128, 192])
def test_fp8_last_row_equal_causal_and_noncausal(mode, dqk):
    # the last query sees every key either way, through the same blocks and masks: bit-exact
    S = 777
    d = W.make_fp8(custom(1, 4, 2, S, dqk), seed=11)
    oc, lc = run_fp8(d, mode, causal=True, return_lse=True)
    on, ln_ = run_fp8(d, mode, causal=False, return_lse=True)
    assert torch.equal(oc[:, S - 1].view(torch.int16), on[:, S - 1].view(torch.int16))
    assert torch.equal(lc[:, :, S - 1], ln_[:, :, S - 1])


@pytest.mark.parametrize("mode", MODES)
def test_fp8_zero_query_closed_forms(mode):
    # Q = 0: every probability is 256 exactly, so O is the mean of the visible V rows and
    # lse = ln(number of visible keys), up to fp32 rounding
    S = 300
    d = W.make_fp8(custom(1, 2, 2, S, 128), seed=5)
    d["q8"] = torch.zeros_like(d["q8"])
    vd = decode_e4m3(d["v8"].numpy())
    for causal in (True, False):
        out, lse = run_fp8(d, mode, causal=causal, return_lse=True)
        got = gpu_select(out)
        n = np.arange(1, S + 1) if causal else np.full(S, S)
        if causal:
            mean = d["v_scale"] * np.cumsum(vd, axis=1) / n[None, :, None, None]
        else:
            mean = np.broadcast_to(d["v_scale"] * vd.mean(axis=1, keepdims=True), got.shape)
        assert np.max(np.abs(got - mean) / (np.abs(mean) + 1e-3)) < 2 ** -7
        assert np.max(np.abs(lse_select(lse) - np.log(n)[None, None, :])) < 1e-5


@pytest.mark.parametrize("name,mode", [("gauss32k", "lean"), ("mistral", "exact"), ("mla", "exact")])
def test_fp8_noncausal_full_size_sampled(name, mode):
    w = W.WORKLOADS[name]
    d = W.make_fp8(w)
    out, lse = run_fp8(d, mode, causal=False, return_lse=True)
    rows = W.sample_rows(w.S, 512).numpy()         # every row sees all S keys
    heads = sorted({0, w.Hq - 1})
    emu, ref, lemu, lref = oracle_fp8(d, mode, heads=heads, rows=rows, causal=False, with_lse=True)
    label = f"{name} {mode} non-causal (rows={len(rows)}, heads={heads})"
    check_fp8(gpu_select(out, heads=heads, rows=rows), emu, ref, label, rows=rows, d=d, mode=mode, heads=heads,
              causal=False)
    check_lse_fp8(lse_select(lse, heads=heads, rows=rows), lemu, lref, mode, label, d=d, rows=rows, heads=heads,
                  causal=False)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("name,mode", [("gauss32k", "lean"), ("mla", "exact")])
def test_fp8_causal_lse_full_size_sampled(name, mode):
    w = W.WORKLOADS[name]
    d = W.make_fp8(w)
    out, lse = run_fp8(d, mode, return_lse=True)
    rows = W.sample_rows_long(w.S, 1024).numpy()
    heads = sorted({0, w.Hq - 1})
    emu, ref, lemu, lref = oracle_fp8(d, mode, heads=heads, rows=rows, with_lse=True)
    check_fp8(gpu_select(out, heads=heads, rows=rows), emu, ref, f"{name} {mode} causal lse call", rows=rows, d=d,
              mode=mode, heads=heads)
    check_lse_fp8(lse_select(lse, heads=heads, rows=rows), lemu, lref, mode, f"{name} {mode} causal", d=d, rows=rows,
                  heads=heads)
    assert bool(torch.isfinite(lse).all())


# ----------------------------------------------------------------------------- BF16

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 1, 128), (2, 4, 2, 129, 128), (1, 4, 1, 333, 192),
                                   (1, 2, 2, 65, 192), (1, 8, 2, 1000, 128)])
def test_bf16_output_and_lse_full_tensor(shape, causal):
    B, Hq, Hkv, S, dqk = shape
    d = W.make_bf16(custom(B, Hq, Hkv, S, dqk), seed=57 + S)
    out, lse = run_bf16(d, causal=causal, return_lse=True)
    ref, lref = oracle_bf16(d, causal=causal, with_lse=True)
    e, er = rel_rms(gpu_select(out), ref), row_rel_rms(gpu_select(out), ref)
    dl = np.abs(lse_select(lse) - lref).max()
    print(f"[parity] bf16 {shape} causal={causal}: vs fp64 {e:.2e}, per row max {er.max():.2e}, lse max |diff| {dl:.2e}")
    assert np.all(np.isfinite(gpu_select(out))) and e <= TOL_BF16 and er.max() <= TOL_BF16_ROW
    assert dl <= TOL_LSE_BF16


def test_bf16_last_row_equal_causal_and_noncausal():
    S = 777
    d = W.make_bf16(custom(1, 4, 2, S, 128), seed=12)
    oc, lc = run_bf16(d, causal=True, return_lse=True)
    on, ln_ = run_bf16(d, causal=False, return_lse=True)
    assert torch.equal(oc[:, S - 1].view(torch.int16), on[:, S - 1].view(torch.int16))
    assert torch.equal(lc[:, :, S - 1], ln_[:, :, S - 1])


@pytest.mark.parametrize("name", ["qwen", "mla"])
def test_bf16_noncausal_full_size_sampled(name):
    w = W.WORKLOADS[name]
    d = W.make_bf16(w)
    out, lse = run_bf16(d, causal=False, return_lse=True)
    rows = W.sample_rows(w.S, 512).numpy()
    heads = sorted({0, w.Hq - 1})
    ref, lref = oracle_bf16(d, heads=heads, rows=rows, causal=False, with_lse=True)
    got = gpu_select(out, heads=heads, rows=rows)
    e, er = rel_rms(got, ref), row_rel_rms(got, ref)
    dl = np.abs(lse_select(lse, heads=heads, rows=rows) - lref).max()
    print(f"[parity] bf16 {name} non-causal: vs fp64 {e:.2e}, per row max {er.max():.2e}, lse max |diff| {dl:.2e}")
    assert e <= TOL_BF16 and er.max() <= TOL_BF16_ROW and dl <= TOL_LSE_BF16 and bool(torch.isfinite(out).all())
