"""Hadamard rotation of Q and K ahead of their per-tensor FP8 quantisation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[MTP] section "How accurate is ZYFA's FP8 attention?": most of the end-to-end
FP8 error comes from quantising Q, K and V, and rotating Q and K by a Hadamard
matrix cuts the input error to about half, at about 0.1% of the attention time.
The pages give no further detail; the readings taken here:

* the orthonormal Sylvester-Hadamard matrix H_n[i, j] = (-1)^popcount(i & j) /
  sqrt(n) multiplies every (token, head) vector along the head dimension, x -> x H;
* block size n = 128 for d = 128; d = 192 is not a power of two, so it is split
  into three blocks of n = 64 (a block-diagonal rotation, still orthogonal);
* then the per-tensor quantisation the inputs already use: scale = amax / 448 of
  the rotated tensor (1 if it is all zero), codes = e4m3 RNE(x / scale),
  saturating.

H is orthogonal, so (Q H)(K H)^T = Q K^T: the scores are unchanged in exact
arithmetic and only the quantisation error moves (spreading an outlier channel
over all dimensions of its block lowers amax relative to the typical value).

Pins (``tests/test_oracle_rotate.py``): H H^T = n I; the closed form against the
recursive construction; worked vectors; norm preservation; fp64 attention
invariance; and the pages' claim itself, lower attention error after rotation on
inputs with outlier channels.
"""
import numpy as np

from .e4m3 import E4M3_MAX, encode_e4m3_rne


def hadamard(n):
    """Unnormalised Sylvester-Hadamard matrix of order n (a power of two): H_1 = [1],
    H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != n:
        raise ValueError(f"order {n} is not a power of two")
    return h


def block_size(d):
    """Rotation block along the head dimension: 128 when it divides d, else 64."""
    n = 128 if d % 128 == 0 else 64
    if d % n:
        raise ValueError(f"head dimension {d} is not a multiple of 64")
    return n


def rotate(x):
    """x (..., d) -> each block of n consecutive dimensions times H_n / sqrt(n), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    n = block_size(d)
    h = hadamard(n) / np.sqrt(n)
    return (x.reshape(x.shape[:-1] + (d // n, n)) @ h).reshape(x.shape)


def quantize_per_tensor(y):
    """Per-tensor e4m3 quantisation: (codes uint8, scale).  scale = amax/448 as an fp32
    number (1 when amax = 0); codes = RNE(y / scale), saturating at +-448."""
    y = np.asarray(y, dtype=np.float64)
    amax = float(np.max(np.abs(y))) if y.size else 0.0
    scale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    return encode_e4m3_rne(y / scale).astype(np.uint8), scale


def rotate_quantize(x):
    """Hadamard-rotate then quantise per tensor: (codes, scale)."""
    return quantize_per_tensor(rotate(x))
