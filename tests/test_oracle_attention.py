"""Pins of the fp64 attention definition (oracle/attention64.py).

Checked against brute force written as pure-Python loops on tiny shapes and
against closed forms / invariants of causal softmax attention (the operation of
[KG-en] "Breaking the FP8 Attention Bottleneck on AMD MI355X: How Zyphra ZYFA
Unleashes Performance", §"Application Boundaries and Engineering Decisions":
causal forward prefill with equal query and key lengths).
"""
import math

import numpy as np
import pytest

from oracle.attention64 import attention_fp64, attention_weights_fp64, lse_fp64, rel_rms


def brute_force(q, k, v, sm, causal):
    """Pure-Python loops; grouped KV heads by consecutive groups."""
    B, S, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    out = np.zeros((B, S, Hq, dv))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(S):
                js = range(i + 1) if causal else range(S)
                logits = []
                for j in js:
                    acc = 0.0
                    for c in range(dqk):
                        acc += float(q[b, i, h, c]) * float(k[b, j, g, c])
                    logits.append(sm * acc)
                mx = max(logits)
                ws = [math.exp(x - mx) for x in logits]
                tot = sum(ws)
                for e in range(dv):
                    out[b, i, h, e] = sum(w * float(v[b, j, g, e]) for w, j in zip(ws, js)) / tot
    return out


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 9, 4, 2, 5, 3), (2, 12, 2, 2, 4, 6), (1, 7, 3, 1, 3, 4)])
def test_matches_brute_force(shape, causal):
    B, S, Hq, Hkv, dqk, dv = shape
    rng = np.random.default_rng(sum(shape))
    q = rng.standard_normal((B, S, Hq, dqk)) * 2
    k = rng.standard_normal((B, S, Hkv, dqk))
    v = rng.standard_normal((B, S, Hkv, dv))
    sm = 0.7
    ours = attention_fp64(q, k, v, sm_scale=sm, causal=causal, chunk=4)
    ref = brute_force(q, k, v, sm, causal)
    assert np.max(np.abs(ours - ref)) < 1e-12


def _rand(S=40, Hq=4, Hkv=2, dqk=16, dv=8, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((1, S, Hq, dqk)), rng.standard_normal((1, S, Hkv, dqk)),
            rng.standard_normal((1, S, Hkv, dv)))


def test_weights_rows_sum_to_one_and_are_causal():
    q, k, _ = _rand()
    w = attention_weights_fp64(q, k)
    assert np.allclose(w.sum(axis=-1), 1.0, atol=1e-14, rtol=0)
    assert np.all(np.triu(w[0, 0], 1) == 0)


def test_row0_is_v0_and_zero_query_gives_prefix_mean():
    q, k, v = _rand()
    o = attention_fp64(q, k, v)
    for h in range(4):
        assert np.allclose(o[0, 0, h], v[0, 0, h // 2], atol=1e-15, rtol=0)
    o0 = attention_fp64(np.zeros_like(q), k, v)
    for h in range(4):
        pm = np.cumsum(v[0, :, h // 2], axis=0) / np.arange(1, 41)[:, None]
        assert np.max(np.abs(o0[0, :, h] - pm)) < 1e-14


def test_linear_in_v_and_gqa_equals_repeated_mha():
    q, k, v = _rand()
    o = attention_fp64(q, k, v)
    assert np.max(np.abs(attention_fp64(q, k, 3.5 * v) - 3.5 * o)) < 1e-13
    k_rep = np.repeat(k, 2, axis=2)
    v_rep = np.repeat(v, 2, axis=2)
    assert np.max(np.abs(attention_fp64(q, k_rep, v_rep) - o)) < 1e-15


def test_last_causal_row_equals_noncausal_last_row_and_row_subsets():
    q, k, v = _rand(S=33)
    oc = attention_fp64(q, k, v, causal=True)
    on = attention_fp64(q, k, v, causal=False)
    assert np.max(np.abs(oc[0, -1] - on[0, -1])) < 1e-14
    rows = np.array([0, 5, 17, 32])
    assert np.array_equal(attention_fp64(q, k, v, rows=rows), oc[:, rows])


def test_rel_rms():
    a = np.array([3.0, 4.0])
    assert rel_rms(a * 1.01, a) == pytest.approx(0.01)


def brute_force_lse(q, k, sm, causal):
    """Pure-Python log-sum-exp of each row's logits, (B, Hq, S)."""
    B, S, Hq, dqk = q.shape
    Hkv = k.shape[2]
    out = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(S):
                logits = [sm * sum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(dqk))
                          for j in (range(i + 1) if causal else range(S))]
                out[b, h, i] = math.log(sum(math.exp(x) for x in logits))
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_lse_matches_brute_force(causal):
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 11, 4, 5)) * 1.5
    k = rng.standard_normal((2, 11, 2, 5))
    ours = lse_fp64(q, k, sm_scale=0.6, causal=causal, chunk=3)
    assert np.max(np.abs(ours - brute_force_lse(q, k, 0.6, causal))) < 1e-12


def test_lse_closed_forms():
    # row 0 of a causal call sees one key: lse = its logit; zero queries: lse = ln(#keys)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 6, 2, 4))
    k = rng.standard_normal((1, 6, 1, 4))
    lse = lse_fp64(q, k, sm_scale=0.5)
    assert np.allclose(lse[0, :, 0], 0.5 * (q[0, 0] @ k[0, 0, 0]), atol=1e-14)
    z = lse_fp64(np.zeros_like(q), k)
    assert np.allclose(z[0, 0], np.log(np.arange(1, 7)), atol=1e-14)
    assert np.allclose(lse_fp64(np.zeros_like(q), k, causal=False), np.log(6.0), atol=1e-14)


# ------------------------------------------------- unequal query and key lengths

def brute_force_unequal(q, k, v, sm, causal):
    """Pure-Python loops: query i of Sq sees keys j <= i + Sk - Sq (causal) or all Sk keys;
    a query that sees no key gets 0 and a log-sum-exp of -inf."""
    B, Sq, Hq, dqk = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Sq, Hq, v.shape[3]))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Sq):
                js = [j for j in range(Sk) if (not causal) or j <= i + Sk - Sq]
                if not js:
                    continue
                logits = [sm * sum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(dqk)) for j in js]
                m = max(logits)
                e = [math.exp(x - m) for x in logits]
                tot = sum(e)
                lse[b, h, i] = m + math.log(tot)
                for c in range(v.shape[3]):
                    out[b, i, h, c] = sum(e[t] * float(v[b, j, g, c]) for t, j in enumerate(js)) / tot
    return out, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Sq,Sk", [(5, 12), (12, 5), (7, 7), (1, 9)])
def test_unequal_lengths_match_brute_force(Sq, Sk, causal):
    rng = np.random.default_rng(Sq * 31 + Sk)
    q = rng.standard_normal((1, Sq, 4, 6))
    k = rng.standard_normal((1, Sk, 2, 6))
    v = rng.standard_normal((1, Sk, 2, 3))
    ref_o, ref_l = brute_force_unequal(q, k, v, 0.7, causal)
    o = attention_fp64(q, k, v, sm_scale=0.7, causal=causal, chunk=4)
    l = lse_fp64(q, k, sm_scale=0.7, causal=causal, chunk=4)
    assert np.max(np.abs(o - ref_o)) < 1e-12
    assert np.array_equal(np.isinf(l), np.isinf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.max(np.abs(l[fin] - ref_l[fin])) < 1e-12


def test_unequal_causal_is_the_tail_of_the_full_problem():
    # Bottom-right alignment: Sq queries against Sk >= Sq keys are the last Sq rows of the
    # equal-length causal problem, whatever the earlier query rows hold.
    rng = np.random.default_rng(8)
    Sk, Sq = 40, 13
    qf = rng.standard_normal((2, Sk, 4, 8))
    k = rng.standard_normal((2, Sk, 2, 8))
    v = rng.standard_normal((2, Sk, 2, 8))
    full = attention_fp64(qf, k, v)
    tail = attention_fp64(qf[:, Sk - Sq:], k, v)
    assert np.max(np.abs(tail - full[:, Sk - Sq:])) < 1e-13
    assert np.max(np.abs(lse_fp64(qf[:, Sk - Sq:], k) - lse_fp64(qf, k)[:, :, Sk - Sq:])) < 1e-12
    # more queries than keys: the first Sq - Sk rows see nothing
    o = attention_fp64(rng.standard_normal((1, 9, 2, 8)), k[:1, :4], v[:1, :4])
    assert np.all(o[:, :5] == 0) and np.all(np.abs(o[:, 5:]) > 0)
