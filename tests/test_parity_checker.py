"""CPU checks of the per-row parity checker (tests/parity.py) and of the oracle's list of
ambiguous rounding decisions (oracle.emulate.rounding_alternatives) that it relies on.

The checker must pass an output that differs from the emulation only by bf16 output
rounding and by alternative roundings of ambiguous probabilities, and must fail an output
with a real error confined to one long row, or spread thinly over every row."""
import math

import numpy as np
import pytest

from parity import KAPPA, ROW_BASE, check_rows, explain_by_flips, row_rel_rms
from fp8_causal_prefill_tiled_amd import workloads as W
from oracle.attention64 import kv_head
from oracle.e4m3 import bf16_rne, decode_e4m3, encode_e4m3_rne
from oracle.emulate import emulate_fp8, rounding_alternatives

S = 4096


@pytest.fixture(scope="module")
def problem():
    w = W.Workload("checker", 1, 2, 1, S, 128, 128)
    d = W.make_fp8(w, seed=4242)
    rows = W.sample_rows_long(S, 160).numpy()
    out = {}
    for mode in ("exact", "lean"):
        out[mode] = emulate_fp8(d["q8"].numpy(), d["k8"].numpy(), d["v8"].numpy(), d["q_scale"], d["k_scale"],
                                d["v_scale"], p_mode=mode, rows=rows)
    return d, rows, out


def _bf16(x):
    return bf16_rne(x.astype(np.float32)).astype(np.float64)


def _long_row(rows):
    return int(np.flatnonzero(rows >= S // 2)[5])


@pytest.mark.parametrize("mode", ["exact", "lean"])
def test_bf16_rounded_emulation_passes(problem, mode):
    d, rows, out = problem
    e = check_rows(_bf16(out[mode]), out[mode], "bf16 only", rows=rows, d=d, mode=mode)
    assert e.max() < 3e-3


@pytest.mark.parametrize("mode", ["exact", "lean"])
def test_planted_alternative_rounding_is_explained(problem, mode):
    d, rows, out = problem
    ri = _long_row(rows)
    info = rounding_alternatives(d["q8"].numpy(), d["k8"].numpy(), d["v8"].numpy(), d["q_scale"], d["k_scale"],
                                 d["v_scale"], p_mode=mode, i=int(rows[ri]), h=1, kappa=KAPPA)
    assert np.allclose(info["out"], out[mode][0, ri, 1], rtol=0, atol=1e-12)
    # the heaviest ambiguous key takes its other code
    j, walt = max(info["alt"], key=lambda a: info["weight"][a[0]])
    W_ = info["weight"].copy()
    W_[j] = walt
    flipped = W_ @ info["vhat"] / W_.sum()
    got = _bf16(out[mode]).copy()
    got[0, ri, 1] = _bf16(flipped)
    check_rows(got, out[mode], "planted flip", rows=rows, d=d, mode=mode)
    res, used = explain_by_flips(got[0, ri, 1], info)
    assert res <= ROW_BASE and j in used


@pytest.mark.parametrize("mode", ["exact", "lean"])
@pytest.mark.parametrize("kind", ["scale", "direction"])
def test_two_percent_error_in_one_long_row_fails(problem, mode, kind):
    d, rows, out = problem
    ri = _long_row(rows)
    got = _bf16(out[mode]).copy()
    o = out[mode][0, ri, 0]
    if kind == "scale":
        got[0, ri, 0] = o * 1.02
    else:
        u = np.random.default_rng(1).standard_normal(o.shape)
        got[0, ri, 0] = o + 0.02 * np.linalg.norm(o) * u / np.linalg.norm(u)
    # the whole-sample figure does not see it ...
    assert np.sqrt(np.sum((got - out[mode]) ** 2) / np.sum(out[mode] ** 2)) < 5e-3
    # ... the per-row check does
    with pytest.raises(AssertionError, match="not explained"):
        check_rows(got, out[mode], "perturbed row", rows=rows, d=d, mode=mode)


def test_thin_error_on_every_row_fails_the_median(problem):
    d, rows, out = problem
    o = out["lean"]
    u = np.random.default_rng(2).standard_normal(o.shape)
    u *= np.linalg.norm(o, axis=-1, keepdims=True) / np.linalg.norm(u, axis=-1, keepdims=True)
    got = _bf16(o + 4e-3 * u)
    assert row_rel_rms(got, o).max() < ROW_BASE
    with pytest.raises(AssertionError, match="median"):
        check_rows(got, o, "thin error", rows=rows, d=d, mode="lean")


# ------------------------------------------------------------ rounding_alternatives pins

def _brute_alternatives(q8, k8, qs, ks, mode, i, h, kappa, grid=401):
    """Pure-Python loops: every key's rounding under score shifts sampled across [-eps, eps]."""
    B, S_, Hq, d = q8.shape
    g = kv_head(h, Hq, k8.shape[2])
    C = qs * ks / math.sqrt(d) * math.log2(math.e)
    A = float(np.float32(8.0 * C))
    qd = [float(x) for x in decode_e4m3(q8[0, i, h])]
    n = i + 1
    s, eps = [], []
    for j in range(n):
        kd = [float(x) for x in decode_e4m3(k8[0, j, g])]
        s.append(math.fsum(a * b for a, b in zip(qd, kd)))
        eps.append(kappa * C * sum(max(abs(qd[c] * kd[c]) for c in range(m, m + 64)) for m in range(0, d, 64)))
    res = {}
    for j in range(n):
        blk = j // 64
        M = math.ceil(max(s[jj] * C for jj in range(64 * blk, min(n, 64 * blk + 64))))
        vals = set()
        for u in range(grid):
            dt = eps[j] * (2.0 * u / (grid - 1) - 1.0)
            if mode == "exact":
                vals.add(float(decode_e4m3(encode_e4m3_rne(2.0 ** (s[j] * C + dt - M + 8.0)))))
            else:
                code = min(max(round(A * s[j] + 120.0 - 8.0 * M + 8.0 * dt), 0), 126)
                vals.add(float(decode_e4m3(np.uint8(code))))
        res[j] = (vals, M)
    return res


@pytest.mark.parametrize("mode", ["exact", "lean"])
def test_alternatives_match_brute_force(mode):
    w = W.Workload("alt", 1, 2, 2, 200, 128, 128)
    d = W.make_fp8(w, seed=91)
    q8, k8 = d["q8"].numpy(), d["k8"].numpy()
    i, h, kappa = 190, 1, 2.0 ** -6         # a large kappa, so that many keys are ambiguous
    info = rounding_alternatives(q8, k8, d["v8"].numpy(), d["q_scale"], d["k_scale"], d["v_scale"], p_mode=mode,
                                 i=i, h=h, kappa=kappa)
    brute = _brute_alternatives(q8, k8, d["q_scale"], d["k_scale"], mode, i, h, kappa)
    R = max(M for _, M in brute.values())
    alt = {}
    for j, wa in info["alt"]:
        alt.setdefault(j, set()).add(wa)
    n_amb = 0
    for j, (vals, M) in brute.items():
        f = 2.0 ** (M - R)
        base = info["weight"][j] / f
        assert base in vals, (j, base, vals)
        want = {v * f for v in vals - {base}}
        got = alt.get(j, set())
        # sampling may miss an alternative reachable only at the very ends of the interval
        assert want <= got and len(got) <= 2, (j, want, got)
        n_amb += bool(got)
    assert n_amb >= 5


def test_no_alternatives_at_zero_kappa():
    w = W.Workload("alt0", 1, 1, 1, 300, 192, 128)
    d = W.make_fp8(w, seed=92)
    for mode in ("exact", "lean"):
        info = rounding_alternatives(d["q8"].numpy(), d["k8"].numpy(), d["v8"].numpy(), d["q_scale"],
                                     d["k_scale"], d["v_scale"], p_mode=mode, i=299, kappa=0.0)
        assert info["alt"] == []
