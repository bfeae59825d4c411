"""Storage formats read and written by the classifier head (oracle's own code).

* bfloat16: the upper 16 bits of an IEEE binary32.
* OCP FP8 E4M3FN (the FP8 E4M3 classifier-weight format of ELMO, ai.info
  summary, Key Contributions and Methodology): 1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF are NaN, largest finite
  value 448, smallest subnormal 2^-9.

Encoding (used by the oracle for the SGD writeback) rounds to nearest with
ties to even and keeps the sign of zero, as IEEE rounding does; FP8 saturates
finite overflow to +-448, bfloat16 is encoded for finite values within its range.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_fp8_e4m3fn(codes) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return sign * v


FP8_MAX = 448.0


def encode_fp8_e4m3fn(x) -> np.ndarray:
    """float64 -> E4M3FN code: nearest, ties to even, saturating, sign of zero kept."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), FP8_MAX)
    # quantum of the binade that holds a: 2^(e-3) for normals (e >= -6), 2^-9 below
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                    # unbiased exponent, clamped to the subnormal floor
    q = np.exp2((e - 3).astype(np.float64))
    r = np.rint(a / q) * q                        # np.rint: round half to even
    r = np.minimum(r, FP8_MAX)
    # encode r exactly
    _, ex2 = np.frexp(r)
    e2 = ex2 - 1
    is_norm = r >= 2.0 ** -6
    e_field = np.where(is_norm, e2 + 7, 0)
    m_field = np.where(is_norm, np.rint((r / np.exp2(e2.astype(np.float64)) - 1.0) * 8.0),
                       np.rint(r / 2.0 ** -9))
    with np.errstate(invalid="ignore"):          # NaN lanes are overwritten below
        code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = code | (neg.astype(np.int64) << 7)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def encode_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit pattern: nearest, ties to even, sign of zero kept (finite values
    of magnitude up to the largest bf16; subnormals on the 2^-133 grid)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > BF16_MAX):
        raise ValueError("encode_bf16 takes finite values within the bf16 range")
    neg = np.signbit(x)
    a = np.abs(x)
    # quantum of the binade that holds a: 8 significant bits, so 2^(e-7) for a in
    # [2^e, 2^(e+1)), e >= -126; 2^-133 below the smallest normal
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -126)
    q = np.exp2((e - 7).astype(np.float64))
    r = np.rint(a / q) * q                        # np.rint: round half to even
    if np.any(r > BF16_MAX):
        raise ValueError("value rounds past the largest bf16")
    # every bf16 value is a float32 value: its upper 16 bits are the pattern
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits | (neg.astype(np.uint16) << np.uint16(15))
