"""Pins of the oracle's storage-format code against torch's library conversions
and against the independent encoder of the input generator."""
import numpy as np
import pytest
import torch

from oracle.formats import FP8_MAX, decode_bf16, decode_fp8_e4m3fn, encode_fp8_e4m3fn
from workloads.gen import _fp8_bytes, _bf16_bits


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_fp8_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.nanmax(ours) == 448.0 and ours[1] == 2.0 ** -9
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_fp8_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(encode_fp8_e4m3fn(decode_fp8_e4m3fn(codes)), codes)


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    pos = decode_fp8_e4m3fn(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2                      # exact ties: round to the even code
    # torch casts float64 -> float32 before rounding to fp8, so every input here is
    # float32-exact (its own double rounding then equals one correct rounding)
    m32 = mids.astype(np.float32)
    near = np.concatenate([np.nextafter(m32, np.float32(np.inf)),
                           np.nextafter(m32, np.float32(-np.inf))]).astype(np.float64)
    rand = (rng.normal(0, 1, 200000) * np.exp2(rng.integers(-12, 9, 200000))).astype(np.float32).astype(np.float64)
    x = np.concatenate([pos, mids, near, rand, -mids, -rand])
    x = x[np.abs(x) <= 464.0]                             # torch turns |x| > 464 into NaN
    ours = encode_fp8_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_encode_saturates_and_keeps_signed_zero():
    x = np.array([448.0, 449.0, 500.0, 1e30, -1e30, -470.0])
    assert encode_fp8_e4m3fn(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert encode_fp8_e4m3fn(np.array([-1e-6, 1e-6, -0.0])).tolist() == [0x80, 0x00, 0x80]
    assert encode_fp8_e4m3fn(np.array([np.nan])).tolist() == [0x7F]
    assert FP8_MAX == 448.0


def test_fp8_oracle_encoder_agrees_with_generator_encoder():
    # two independent implementations (frexp/rint arithmetic vs nearest-code table search)
    rng = np.random.default_rng(1)
    x = rng.normal(0, 0.05, 500000)
    a = encode_fp8_e4m3fn(x)
    b = _fp8_bytes(x)
    zero = decode_fp8_e4m3fn(a) == 0
    assert np.array_equal(a[~zero], b[~zero])
    assert np.all(decode_fp8_e4m3fn(b[zero]) == 0)


def test_generator_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.normal(0, 1, 100000) * np.exp2(rng.integers(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_bf16_bits(x), ref)


def test_generator_fp8_encoder_matches_nearest_even_table():
    """The input generator's fast E4M3FN rounding equals a brute-force nearest-value
    search over the 127 finite codes with ties to the even code, saturating at 448
    (including every code, every midpoint and its float32 neighbours)."""
    from workloads.gen import _fp8_bytes, fp8_e4m3fn_values
    vals = fp8_e4m3fn_values()[:127]
    rng = np.random.default_rng(0)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([np.concatenate([rng.normal(0, s, 4000) for s in (0.01, 0.05, 1.0, 100.0, 500.0)]).astype(np.float32),
                        vals.astype(np.float32), -vals.astype(np.float32), mids, -mids,
                        np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                        np.float32([448, 449, 463.9, 464, 465, 1e6, -1e6, 0.0, 1e-30])])
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - vals[None, :])
    cand = d == d.min(1, keepdims=True)
    even = np.arange(127)[None, :] % 2 == 0
    idx = np.where(cand.sum(1) > 1, np.argmax(cand & even, axis=1), np.argmin(d, axis=1))
    ref = idx.astype(np.uint8) | ((np.signbit(x) & (idx != 0)).astype(np.uint8) << 7)
    assert np.array_equal(_fp8_bytes(x), ref)


def _bf16_nearest_even_by_search(x):
    """Brute force: the nearest finite bf16 value by a search of the sorted grid of every
    non-negative finite pattern, ties to the even pattern, sign applied afterwards."""
    bits = np.arange(0x7F80, dtype=np.uint32).astype(np.uint16)      # +0 .. largest finite
    vals = decode_bf16(bits)
    a = np.abs(x)
    hi = np.searchsorted(vals, a, side="left").clip(0, len(vals) - 1)
    lo = (hi - 1).clip(0, None)
    dlo, dhi = np.abs(a - vals[lo]), np.abs(vals[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return bits[pick] | (np.signbit(x).astype(np.uint16) << np.uint16(15))


def test_bf16_encode_matches_nearest_even_search_and_torch():
    from oracle.formats import encode_bf16
    rng = np.random.default_rng(5)
    grid = decode_bf16(np.arange(0x7F80, dtype=np.uint32).astype(np.uint16))
    mids = (grid[:-1] + grid[1:]) / 2                        # exact ties
    x = np.concatenate([grid[::7], mids[::5], np.nextafter(mids[::5], 0.0), np.nextafter(mids[::5], np.inf),
                        rng.normal(0, 1, 100000) * np.exp2(rng.integers(-130, 120, 100000)),
                        rng.normal(0, 0.05, 100000)])
    x = np.concatenate([x, -x[::3]])
    assert np.array_equal(encode_bf16(x), _bf16_nearest_even_by_search(x))
    # float32-exact inputs: one correct rounding, as torch's float32 -> bfloat16 cast
    x32 = x.astype(np.float32)
    x32 = x32[np.isfinite(x32)].astype(np.float64)
    ref = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(encode_bf16(x32), ref)
    assert encode_bf16(np.array([-0.0, 0.0])).tolist() == [0x8000, 0x0000]
    with pytest.raises(ValueError):
        encode_bf16(np.array([np.inf]))
