"""Pins of the stochastic-rounding oracle (ELMO, ai.info summary: stochastic rounding of the
classifier weights in the SGD update): the generator against its published known-answer
vectors, and the rounding rule against brute force, closed-form frequencies and its
unbiasedness."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle.formats import decode_fp8_e4m3fn
from oracle.philox import philox4x32
from oracle.stochastic import FP8_MAX, decode, encode, sgd_sr, sr_round, uniform16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")


def test_philox_known_answers():
    kat = json.load(open(GOLDEN))
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["output"]]
        assert [int(x) for x in philox4x32(ctr, key)] == want


def test_philox_vectorized_matches_scalar_calls():
    rng = np.random.default_rng(0)
    ctr = rng.integers(0, 2 ** 32, size=(16, 4), dtype=np.uint64)
    key = rng.integers(0, 2 ** 32, size=2, dtype=np.uint64)
    batch = philox4x32(ctr, key)
    for i in range(16):
        assert np.array_equal(batch[i], philox4x32(ctr[i], key))


def test_uniform16_takes_half_words_in_order():
    v, seed = 123456789012, 0xDEADBEEF12345678
    words = philox4x32([1, v & 0xFFFFFFFF, v >> 32, 0], [seed & 0xFFFFFFFF, seed >> 32])
    halves = []
    for w in words:
        halves += [int(w) & 0xFFFF, int(w) >> 16]
    u = uniform16(np.full(8, v), np.arange(8, 16), seed)
    assert np.array_equal(u * 65536, np.array(halves, dtype=np.float64))


def _grid_brute(fmt):
    codes = np.arange(256) if fmt == "fp8" else np.arange(0, 65536, 7)
    vals = decode(codes.astype(np.uint8 if fmt == "fp8" else np.uint16), fmt)
    return np.sort(vals[np.isfinite(vals)])


@pytest.mark.parametrize("fmt", ["fp8", "bf16"])
def test_grid_values_are_fixed_points(fmt):
    g = _grid_brute(fmt)
    rng = np.random.default_rng(1)
    out = sr_round(g, rng.random(g.shape), fmt)
    assert np.array_equal(out, g + 0.0)


def test_result_is_a_neighbour_found_by_linear_scan():
    grid = _grid_brute("fp8")
    rng = np.random.default_rng(2)
    y = rng.uniform(-500, 500, 3000) * rng.choice([1e-3, 1e-1, 1.0], 3000)
    u = rng.random(3000)
    out = sr_round(y, u, "fp8")
    for yi, oi in zip(np.clip(y, -FP8_MAX, FP8_MAX), out):
        below = grid[grid <= yi].max()
        above = grid[grid >= yi].min()
        assert oi in (below + 0.0, above + 0.0)


def test_up_count_over_all_uniforms_is_closed_form():
    # with u = k / 2^16 for every k, y rounds up for exactly ceil(f 2^16) values of k,
    # f = (y - lo) / (hi - lo)
    k = np.arange(65536) / 65536.0
    for lo, hi, f in [(0.28125, 0.3125, 0.6), (-0.3125, -0.28125, 0.25), (0.0, 2.0 ** -9, 0.3),
                      (416.0, 448.0, 0.999), (1.0, 1.125, 1.0 / 65536)]:
        y = lo + f * (hi - lo)
        out = sr_round(np.full(k.shape, y), k, "fp8")
        assert set(np.unique(out)) <= {lo + 0.0, hi + 0.0}
        assert np.count_nonzero(out == hi) == int(np.ceil(f * 65536 - 1e-9))


def test_unbiased_over_seeds():
    rng = np.random.default_rng(3)
    y = rng.uniform(-2, 2, 64)
    seeds = np.arange(4000)
    acc = np.zeros_like(y)
    for s in seeds:
        acc += sr_round(y, uniform16(np.arange(64), np.zeros(64, dtype=np.int64), int(s) * 7919), "fp8")
    mean = acc / len(seeds)
    g = _grid_brute("fp8")
    step = np.array([g[g >= yi].min() - g[g <= yi].max() for yi in y])
    # binomial standard error of the mean: step * sqrt(f(1-f) / n) <= step / (2 sqrt(n))
    assert np.all(np.abs(mean - y) <= 5 * step / (2 * np.sqrt(len(seeds))) + step / 65536)


def test_saturation_and_signed_zero():
    out = sr_round(np.array([1000.0, -1000.0, 448.0, -448.0]), np.array([0.1, 0.9, 0.5, 0.5]), "fp8")
    assert list(out) == [448.0, -448.0, 448.0, -448.0]
    z = sr_round(np.array([-1e-5, 1e-5]), np.array([0.99, 0.99]), "fp8")
    assert np.all(z == 0) and not np.any(np.signbit(z))
    assert list(encode(z, "fp8")) == [0, 0]


def test_sgd_sr_update_rounds_the_step():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, size=(5, 24)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10                    # no NaN codes
    dE = rng.standard_normal((5, 24))
    items = np.array([3, 1000, 7, 2 ** 33 + 5, 0])
    out = sgd_sr(codes, items, dE, 0.01, 99, "fp8")
    y = np.clip(decode_fp8_e4m3fn(codes) - 0.01 * dE, -FP8_MAX, FP8_MAX)
    g = _grid_brute("fp8")
    vals = decode_fp8_e4m3fn(out)
    for yi, oi in zip(y.ravel(), vals.ravel()):
        assert g[g <= yi].max() <= oi <= g[g >= yi].min()
    # deterministic in (seed, v, d); another seed changes some roundings
    assert np.array_equal(out, sgd_sr(codes, items, dE, 0.01, 99, "fp8"))
    assert not np.array_equal(out, sgd_sr(codes, items, dE, 0.01, 100, "fp8"))
