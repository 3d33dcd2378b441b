"""Pins of oracle/rotate.py (the Hadamard rotation of Q and K before their FP8
quantisation, [MTP] section "How accurate is ZYFA's FP8 attention?") against
facts fixed by the mathematics and by the pages, not by retyping its code."""
import numpy as np
import pytest

from fp8_causal_prefill_tiled_amd import workloads as W
from oracle.attention64 import attention_fp64
from oracle.e4m3 import decode_e4m3
from oracle.rotate import block_size, hadamard, quantize_per_tensor, rotate, rotate_quantize


@pytest.mark.parametrize("n", [1, 2, 4, 64, 128])
def test_hadamard_rows_are_orthogonal(n):
    h = hadamard(n)
    assert np.array_equal(h @ h.T, n * np.eye(n))
    assert set(np.unique(h)) <= {-1.0, 1.0}


@pytest.mark.parametrize("n", [64, 128])
def test_hadamard_closed_form(n):
    # Sylvester order: entry (i, j) is (-1)^(number of bits i and j share)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    pop = np.vectorize(lambda x: bin(int(x)).count("1"))(i & j)
    assert np.array_equal(hadamard(n), np.where(pop % 2 == 0, 1.0, -1.0))


def test_worked_vectors():
    assert np.array_equal(hadamard(2), [[1, 1], [1, -1]])
    assert np.array_equal(hadamard(4)[3], [1, -1, -1, 1])
    e0 = np.zeros(128)
    e0[0] = 1.0
    assert np.allclose(rotate(e0), np.full(128, 1 / np.sqrt(128)), rtol=0, atol=1e-15)
    c = np.full(128, 3.0)   # a constant vector concentrates on dimension 0
    r = rotate(c)
    assert abs(r[0] - 3.0 * np.sqrt(128)) < 1e-12 and np.max(np.abs(r[1:])) < 1e-12
    # d = 192 rotates three 64-blocks independently
    x = np.zeros(192)
    x[64] = 1.0
    r = rotate(x)
    assert np.allclose(r[64:128], 1 / 8) and np.all(r[:64] == 0) and np.all(r[128:] == 0)
    assert block_size(128) == 128 and block_size(192) == 64
    with pytest.raises(ValueError):
        block_size(96)


@pytest.mark.parametrize("d", [128, 192])
def test_rotation_preserves_norms_and_is_invertible(d):
    x = np.random.default_rng(5).standard_normal((7, 3, d))
    r = rotate(x)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.allclose(rotate(r), x, atol=1e-12)   # the normalised Sylvester matrix is its own inverse


@pytest.mark.parametrize("d,hq,hkv", [(128, 4, 2), (192, 2, 2)])
def test_attention_is_invariant_under_the_rotation(d, hq, hkv):
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 80, hq, d))
    k = rng.standard_normal((1, 80, hkv, d))
    v = rng.standard_normal((1, 80, hkv, 128))
    a = attention_fp64(q, k, v)
    b = attention_fp64(rotate(q), rotate(k), v)
    assert np.max(np.abs(a - b)) < 1e-12


def test_quantisation_conventions():
    codes, scale = quantize_per_tensor(np.zeros((2, 3)))
    assert scale == 1.0 and not codes.any()
    y = np.array([-896.0, 1.0, 0.0, 448.0 * 2])
    codes, scale = quantize_per_tensor(y)
    assert scale == 2.0
    assert np.array_equal(decode_e4m3(codes), [-448.0, 0.5, 0.0, 448.0])


def _attention_error(w, rotate_first):
    q, k, v = (t.numpy().astype(np.float64) for t in W.draw_fp32(w))
    ref = attention_fp64(q, k, v)
    quant = rotate_quantize if rotate_first else quantize_per_tensor
    (q8, qs), (k8, ks) = quant(q), quant(k)
    out = attention_fp64(decode_e4m3(q8) * qs, decode_e4m3(k8) * ks, v)
    return np.sqrt(np.sum((out - ref) ** 2) / np.sum(ref ** 2))


def test_rotation_cuts_the_input_error_with_outlier_channels():
    # The pages report the rotation cutting the input-quantisation error to about a half on a
    # real model; on Mistral-shaped inputs (4 outlier channels x8) it must do at least that.
    w = W.WORKLOADS["mistral"].with_(S=384, Hq=4, Hkv=2)
    assert _attention_error(w, True) < 0.5 * _attention_error(w, False)


def test_rotation_is_neutral_on_gaussian_inputs():
    w = W.WORKLOADS["gauss32k"].with_(S=384, Hq=4, Hkv=4)
    ratio = _attention_error(w, True) / _attention_error(w, False)
    assert 0.9 < ratio < 1.1
