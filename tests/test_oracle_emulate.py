"""Pins of the FP8 method emulation (oracle/emulate.py).

Each pin ties one step of the method, as the pages describe it, to something
other than the emulation itself: the plain definition it reduces to, closed
forms, or bounds that follow from the e4m3 format.  Sources:
[MTP] "Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x Faster",
§"Lean P: one multiply-add instead of an exponential" and §"Per-block scaling
and a rounded row sum"; [KG-zh] (Chinese version of the kg.zhiyong.dev article),
§技术解法 (why the denominator is the sum of rounded probabilities).
"""
import numpy as np
import pytest

from oracle.attention64 import attention_fp64, dequantize, lse_fp64, rel_rms
from oracle.e4m3 import decode_e4m3, encode_e4m3_rne
from oracle.emulate import (emulate_fp8, block_probabilities, encode_probability_lean,
                            encode_probability_exact, LOG2E)


def _codes(shape, rng, sigma=1.0, scale_to=448.0):
    x = rng.standard_normal(shape) * sigma
    s = np.abs(x).max() / scale_to
    return encode_e4m3_rne(x / s), s


def _inputs(S=200, Hq=2, Hkv=2, dqk=32, dv=16, seed=0, sigma_q=1.0):
    rng = np.random.default_rng(seed)
    q8, qs = _codes((1, S, Hq, dqk), rng, sigma_q)
    k8, ks = _codes((1, S, Hkv, dqk), rng)
    v8, vs = _codes((1, S, Hkv, dv), rng)
    return q8, k8, v8, qs, ks, vs


def test_no_rounding_reduces_to_plain_definition():
    q8, k8, v8, qs, ks, vs = _inputs(S=300, Hq=4, Hkv=2)
    ref = attention_fp64(dequantize(q8, qs), dequantize(k8, ks), dequantize(v8, vs))
    emu = emulate_fp8(q8, k8, v8, qs, ks, vs, rounding=False, chunk=64)
    assert rel_rms(emu, ref) < 1e-13


@pytest.mark.parametrize("p_mode", ["exact", "lean"])
def test_zero_query_gives_prefix_mean_exactly(p_mode):
    # All scores 0 -> every block max is 0 -> every p~ = 2^8 = 256 (code 0x78 on both paths),
    # so O_i = v_scale * mean(decode(V8[0..i])).
    q8, k8, v8, qs, ks, vs = _inputs(S=150)
    q8 = np.zeros_like(q8)
    emu = emulate_fp8(q8, k8, v8, qs, ks, vs, p_mode=p_mode)
    vd = decode_e4m3(v8)
    for h in range(2):
        pm = vs * np.cumsum(vd[0, :, h], axis=0) / np.arange(1, 151)[:, None]
        assert np.max(np.abs(emu[0, :, h] - pm)) <= 1e-13 * np.max(np.abs(pm))
    assert encode_probability_exact(8.0) == 0x78 == encode_probability_lean(8.0)


@pytest.mark.parametrize("p_mode", ["exact", "lean"])
def test_row0_is_v0_and_constant_v_is_exact(p_mode):
    q8, k8, v8, qs, ks, vs = _inputs(S=190, sigma_q=3.0)
    emu = emulate_fp8(q8, k8, v8, qs, ks, vs, p_mode=p_mode)
    assert np.array_equal(emu[0, 0], vs * decode_e4m3(v8[0, 0]))
    # Constant V: the output equals that constant only because the denominator is the
    # sum of the same rounded probabilities that multiply V (the rounded row sum).
    ones = np.full_like(v8, 0x38)  # e4m3 1.0
    emu1 = emulate_fp8(q8, k8, ones, qs, ks, 0.75, p_mode=p_mode)
    assert np.max(np.abs(emu1 - 0.75)) < 1e-14


def test_lean_code_law_is_8x_plus_constant():
    # Doubling a value adds 8 to its e4m3 code: at integer exponents Lean P is exact.
    for n in range(-6, 9):
        assert encode_probability_lean(float(n)) == 8 * n + 56 == encode_probability_exact(float(n))
    # between integers it is the chord of 2^x (never below, at most 6.15% above, before rounding)
    y = np.linspace(-5.99, 7.99, 20001)
    chord = 2.0 ** np.floor(y) * (1.0 + (y - np.floor(y)))
    r = chord / 2.0 ** y
    assert r.min() >= 1.0 and r.max() < 1.0615 + 1e-4


@pytest.mark.parametrize("p_mode", ["exact", "lean"])
def test_block_maximum_lands_in_top_binade(p_mode):
    # The per-(row, 64-key block) power of two puts each block's largest probability in (128, 256].
    q8, k8, v8, qs, ks, vs = _inputs(S=256, sigma_q=4.0, seed=3)
    for i in [0, 1, 63, 64, 65, 127, 200, 255]:
        p, M = block_probabilities(q8, k8, qs, ks, p_mode=p_mode, i=i)
        nb = (i + 64) // 64
        assert p.shape[0] == nb
        bmax = p.max(axis=1)
        if p_mode == "exact":
            assert np.all((bmax >= 128) & (bmax <= 256))
        else:
            codes = encode_e4m3_rne(bmax)
            assert np.all((codes >= 112) & (codes <= 120))
        assert np.all(M == np.round(M))


@pytest.mark.parametrize("p_mode,lo,hi", [("exact", 1 - 2.0**-4, 1 + 2.0**-4),
                                          ("lean", 1 / 1.0667, 1.0615 * 1.0625)])
def test_probability_error_bounds(p_mode, lo, hi):
    # Each rounded probability is within the e4m3 half-ulp (exact path) or within the chord
    # bound times half a code step (Lean P) of the true 2^(t - M + 8), for normal values.
    q8, k8, v8, qs, ks, vs = _inputs(S=256, dqk=64, seed=5, sigma_q=2.0)
    sm = 1 / np.sqrt(64)
    qd, kd = decode_e4m3(q8), decode_e4m3(k8)
    for i in [37, 130, 255]:
        p, M = block_probabilities(q8, k8, qs, ks, p_mode=p_mode, i=i)
        t = (qd[0, i, 0] @ kd[0, :i + 1, 0].T) * qs * ks * sm * LOG2E
        nb = p.shape[0]
        tt = np.full(nb * 64, -np.inf)
        tt[:i + 1] = t
        true = np.exp2(tt.reshape(nb, 64) - M[:, None] + 8)
        normal = true >= 2.0 ** -5
        ratio = p[normal] / true[normal]
        assert ratio.min() >= lo - 1e-12 and ratio.max() <= hi + 1e-12


def test_block_order_independence_noncausal():
    # p~ is taken relative to each block's own maximum, so permuting whole 64-key blocks
    # (keys and values together) leaves the non-causal result unchanged.
    q8, k8, v8, qs, ks, vs = _inputs(S=256, seed=7, sigma_q=2.0)
    base = emulate_fp8(q8, k8, v8, qs, ks, vs, causal=False, p_mode="lean")
    perm = np.concatenate([np.arange(64) + 64 * b for b in [2, 0, 3, 1]])
    out = emulate_fp8(q8, k8[:, perm], v8[:, perm], qs, ks, vs, causal=False, p_mode="lean")
    assert np.max(np.abs(out - base)) <= 1e-13 * np.max(np.abs(base))


def test_gqa_equals_repeated_heads():
    q8, k8, v8, qs, ks, vs = _inputs(S=130, Hq=4, Hkv=2, seed=9)
    a = emulate_fp8(q8, k8, v8, qs, ks, vs, p_mode="exact")
    b = emulate_fp8(q8, np.repeat(k8, 2, axis=2), np.repeat(v8, 2, axis=2), qs, ks, vs, p_mode="exact")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("p_mode,cap", [("exact", 0.03), ("lean", 0.035)])
def test_error_vs_fp64_is_at_the_e4m3_level(p_mode, cap):
    # Rounding P to e4m3 (3 mantissa bits) leaves a relative RMS error of order 2^-3/sqrt(12)
    # on the output; it must be present (>1e-3) and bounded.
    q8, k8, v8, qs, ks, vs = _inputs(S=256, dqk=128, dv=128, seed=11)
    ref = attention_fp64(dequantize(q8, qs), dequantize(k8, ks), dequantize(v8, vs))
    e = rel_rms(emulate_fp8(q8, k8, v8, qs, ks, vs, p_mode=p_mode), ref)
    assert 1e-3 < e < cap


# ----------------------------------------------------------------- row log-sum-exp

@pytest.mark.parametrize("causal", [True, False])
def test_lse_without_rounding_is_the_plain_log_sum_exp(causal):
    # Special case that reduces to the definition: with the exact path unrounded, the
    # emulated denominator is sum_j 2^(t_ij), whose log is the fp64 log-sum-exp.
    q8, k8, v8, qs, ks, vs = _inputs(S=200, Hq=4, Hkv=2, seed=13, sigma_q=2.0)
    _, log2L = emulate_fp8(q8, k8, v8, qs, ks, vs, rounding=False, causal=causal, return_lse=True, chunk=48)
    ref = lse_fp64(dequantize(q8, qs), dequantize(k8, ks), causal=causal)      # (B, Hq, S)
    assert np.max(np.abs(np.log(2.0) * log2L.transpose(0, 2, 1) - ref)) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("p_mode,lo,hi", [("exact", 1 - 2.0**-4, 1 + 2.0**-4),
                                          ("lean", 2.0 ** (-1 / 16), 1.0615 * 1.0625)])
def test_lse_of_rounded_weights_within_the_probability_bounds(p_mode, lo, hi, causal):
    # The denominator is a sum of rounded probabilities, each within [lo, hi] of its true
    # value when normal (e4m3 half-ulp on the exact path; chord times half a code step for
    # Lean P, whose low end is 2^(-1/16): a value just below n + 1/16 rounds down to 2^n).
    # Values below 2^-6 can be off by all of themselves, but 64 of them weigh less than
    # 2^-7 of their block's maximum (> 2^7), so the log moves by at most 2^-7 more.
    q8, k8, v8, qs, ks, vs = _inputs(S=300, Hq=2, Hkv=1, dqk=64, seed=17, sigma_q=2.0)
    _, log2L = emulate_fp8(q8, k8, v8, qs, ks, vs, p_mode=p_mode, causal=causal, return_lse=True)
    d = np.log(2.0) * log2L.transpose(0, 2, 1) - lse_fp64(dequantize(q8, qs), dequantize(k8, ks), causal=causal)
    assert d.min() >= np.log(lo) - 2.0 ** -7 and d.max() <= np.log(hi) + 2.0 ** -7
    # the rounding is visible (the bound is not vacuous) and mostly averages out over a row
    assert np.abs(d).max() > 1e-4 and np.abs(d).mean() < 0.05


# ------------------------------------------------- unequal query and key lengths

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Sq,Sk", [(70, 200), (200, 70), (1, 129)])
def test_unequal_lengths_without_rounding_is_the_plain_definition(Sq, Sk, causal):
    rng = np.random.default_rng(Sq + 7 * Sk)
    q8, qs = _codes((1, Sq, 4, 32), rng, 2.0)
    k8, ks = _codes((1, Sk, 2, 32), rng)
    v8, vs = _codes((1, Sk, 2, 16), rng)
    qd, kd, vd = dequantize(q8, qs), dequantize(k8, ks), dequantize(v8, vs)
    emu, log2L = emulate_fp8(q8, k8, v8, qs, ks, vs, rounding=False, causal=causal, return_lse=True, chunk=48)
    assert np.max(np.abs(emu - attention_fp64(qd, kd, vd, causal=causal))) < 1e-12
    ref = lse_fp64(qd, kd, causal=causal)
    got = np.log(2.0) * log2L.transpose(0, 2, 1)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    assert np.max(np.abs(got[fin] - ref[fin])) < 1e-12


@pytest.mark.parametrize("p_mode", ["exact", "lean"])
def test_unequal_causal_emulation_is_the_tail_of_the_full_problem(p_mode):
    # the rounded method too: each row's blocks, exponents and rounded probabilities are the same
    rng = np.random.default_rng(12)
    Sk, Sq = 300, 77
    q8, qs = _codes((1, Sk, 2, 64), rng, 2.0)
    k8, ks = _codes((1, Sk, 1, 64), rng)
    v8, vs = _codes((1, Sk, 1, 32), rng)
    full, lf = emulate_fp8(q8, k8, v8, qs, ks, vs, p_mode=p_mode, return_lse=True)
    tail, lt = emulate_fp8(q8[:, Sk - Sq:], k8, v8, qs, ks, vs, p_mode=p_mode, return_lse=True)
    assert np.max(np.abs(tail - full[:, Sk - Sq:])) <= 1e-13 * np.max(np.abs(full))
    assert np.max(np.abs(lt - lf[:, Sk - Sq:])) < 1e-12


def _floor_closed_form(mode, n=200_000):
    """Relative RMS error floor that rounding every probability to e4m3 leaves in a long row,
    from the format definition alone.

    With the log2 of a probability uniform modulo 1 (scores spread over many binades), its
    rounded value is p (1 + delta(f)), f the fractional part.  Normalising by the sum of the
    rounded values cancels the mean of delta, and for value rows independent of the scores the
    output's relative RMS error is sd(delta) / (1 + mean(delta)).
      exact: the 3-bit mantissa rounded to nearest, m = 2^f -> round(8 m) / 8;
      Lean P: code = rint(8 f + 56) read back as 2^(code//8 - 7) (1 + (code % 8) / 8)."""
    f = (np.arange(n) + 0.5) / n
    m = 2.0 ** f
    if mode == "exact":
        val = np.round(8.0 * m) / 8.0
    else:
        code = np.rint(8.0 * f + 56.0)
        val = 2.0 ** (np.floor(code / 8.0) - 7.0) * (1.0 + (code % 8.0) / 8.0)
    delta = val / m - 1.0
    return float(delta.std() / (1.0 + delta.mean()))


@pytest.mark.parametrize("mode,expected", [("exact", 0.0265), ("lean", 0.0314)])
def test_long_row_error_sits_at_e4m3_floor(mode, expected):
    """The emulation's error against fp64, on long causal rows of a Gaussian workload, is the
    closed-form e4m3 rounding floor (within 5%): the rounding, not anything else, sets it."""
    from fp8_causal_prefill_tiled_amd import workloads as W
    floor = _floor_closed_form(mode)
    assert abs(floor - expected) < 2e-4
    w = W.Workload("floor", 1, 1, 1, 8192, 128, 128)
    d = W.make_fp8(w, seed=555)
    rows = np.sort(np.random.default_rng(0).choice(np.arange(4096, 8192), 256, replace=False))
    q8, k8, v8 = d["q8"].numpy(), d["k8"].numpy(), d["v8"].numpy()
    ref = attention_fp64(dequantize(q8, d["q_scale"]), dequantize(k8, d["k_scale"]),
                         dequantize(v8, d["v_scale"]), rows=rows)
    emu = emulate_fp8(q8, k8, v8, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=mode, rows=rows)
    per_row = np.sqrt(np.sum((emu - ref) ** 2, axis=-1) / np.sum(ref ** 2, axis=-1))
    measured = float(np.sqrt(np.mean(per_row ** 2)))
    assert abs(measured / floor - 1.0) < 0.05, (mode, measured, floor)
