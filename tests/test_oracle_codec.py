"""Pins of the oracle's e4m3fn / bf16 codec against the format definition and torch.

The pages rely on the e4m3 bit pattern growing by 8 per doubling of the value
([MTP] "Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x Faster",
§"Lean P: one multiply-add instead of an exponential").
"""
import numpy as np
import pytest
import torch

from oracle.e4m3 import decode_e4m3, encode_e4m3_rne, bf16_rne, E4M3_MAX


def torch_decode(codes):
    return torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3(codes)
    ref = torch_decode(codes)
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert set(np.nonzero(nan_ours)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours], ref[~nan_ours])


def test_closed_forms():
    # code(2^n) = 8n + 56 for every normal power of two: doubling adds 8 to the code.
    for n in range(-6, 9):
        assert encode_e4m3_rne(2.0 ** n) == 8 * n + 56
        assert decode_e4m3(np.uint8(8 * n + 56)) == 2.0 ** n
    # subnormals k * 2^-9, the largest finite value, signed zero
    for kk in range(1, 8):
        assert decode_e4m3(np.uint8(kk)) == kk * 2.0 ** -9
    assert decode_e4m3(np.uint8(0x7E)) == E4M3_MAX == 448.0
    assert decode_e4m3(np.uint8(0xFE)) == -448.0
    assert decode_e4m3(np.uint8(0x00)) == 0.0 and decode_e4m3(np.uint8(0x80)) == 0.0


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode_e4m3_rne(decode_e4m3(codes)), codes)


def test_encode_matches_torch_rne_random():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000) * 30.0,
        np.ldexp(rng.uniform(1, 2, 50000), rng.integers(-12, 9, 50000)) * rng.choice([-1, 1], 50000),
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3_rne(x), ref)


def test_encode_ties_go_to_even_code_and_saturate():
    vals = decode_e4m3(np.arange(0, 127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2.0
    codes = encode_e4m3_rne(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0, 126)) | (codes == np.arange(1, 127)))
    assert encode_e4m3_rne(1000.0) == 0x7E and encode_e4m3_rne(-1e9) == 0xFE
    assert encode_e4m3_rne(np.nan) == 0x7F


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(300000) * np.exp(rng.uniform(-20, 20, 300000))).astype(np.float32)
    # include exact ties: mantissa low half 0x8000 with both parities of the kept lsb
    u = rng.integers(0, 2**31, 20000, dtype=np.uint64).astype(np.uint32) & np.uint32(0x7FFF0000)
    ties = (u | np.uint32(0x00008000)).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_rne(x), ref)
