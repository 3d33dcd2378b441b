"""OCP FP8 e4m3fn codec and bf16 rounding, written from the format's definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the probability and input format "FP8 e4m3" ([KG-en] §"The Core
Bottleneck"; [MTP] §TL;DR) and rely on one property of its bit pattern: read as
an unsigned integer, doubling a value adds 8 to its code ([MTP] §"Lean P: one
multiply-add instead of an exponential").  The flavour is OCP e4m3fn: exponent
bias 7, 3 mantissa bits, subnormals M*2^-9, no infinities, a single NaN pattern
per sign (S.1111.111), largest finite 448 (a reading: the per-tensor scale
amax/448 used for the inputs fixes the 448 maximum).

Pins (in ``tests/test_oracle_codec.py``): exhaustive comparison with torch's
float8_e4m3fn decode (a library routine), the closed form code(2^n) = 8n + 56,
round-trip identity on all finite codes, and RNE/saturation behaviour.
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7


def decode_e4m3(codes):
    """Value of each e4m3fn byte (uint8 array) as float64; NaN for 0x7F/0xFF."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - E4M3_BIAS)
    subnormal = (m / 8.0) * np.ldexp(1.0, 1 - E4M3_BIAS)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# The 127 non-negative finite values, indexed by their code 0x00..0x7E; the
# code order is the value order, so "nearest, ties to even code" is RNE.
_POS_VALUES = decode_e4m3(np.arange(0, 127, dtype=np.uint8))


def encode_e4m3_rne(x):
    """Round float values to the nearest e4m3fn code, ties to even, saturating.

    |x| >= 448 maps to +-448 (code 0x7E / 0xFE); NaN maps to 0x7F.  Zero and
    negative zero keep their sign bit.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    idx_hi = np.searchsorted(_POS_VALUES, np.minimum(a, E4M3_MAX), side="left")
    idx_hi = np.clip(idx_hi, 0, 126)
    idx_lo = np.clip(idx_hi - 1, 0, 126)
    v_hi = _POS_VALUES[idx_hi]
    v_lo = _POS_VALUES[idx_lo]
    d_hi = v_hi - np.minimum(a, E4M3_MAX)
    d_lo = np.minimum(a, E4M3_MAX) - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (idx_hi % 2 == 0))
    code = np.where(pick_hi, idx_hi, idx_lo).astype(np.int64)
    code = np.where(a >= E4M3_MAX, 126, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def round_to_e4m3(x):
    """RNE-round values to e4m3fn and return them as float64 values."""
    return decode_e4m3(encode_e4m3_rne(x))


def bf16_rne(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Works on the float32 bit pattern: a bf16 is the top 16 bits of a float32.
    Returns float32 values that are exactly representable in bf16.  NaN stays NaN.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), np.float32(np.nan), out)
