"""Stochastic rounding of the SGD writeback (oracle; test infrastructure: only the tests,
smoke() and the bench's CPU baseline use it).

ELMO (ai.info summary: Key Contributions 1, Methodology) keeps the classifier weights in
BF16 or FP8 E4M3 with no higher-precision master copy and rounds each SGD update
stochastically, up or down at random so that small updates survive on average. The pages
fix neither the generator nor the bit budget; the readings are:

* The value to round is y = E_vd - lr dE_vd (FP8: first clamped to [-448, 448], the
  saturating range of E4M3FN).
* lo is the largest and hi the smallest value of the storage format's finite grid with
  lo <= y <= hi. If y is on the grid it is kept. Otherwise y rounds to hi exactly when
  u (hi - lo) < y - lo, for a uniform u in [0, 1): hi with probability (y - lo) / (hi - lo)
  (up to the 2^-16 granularity of u), so the rounding is unbiased.
* u = h / 2^16, h the 16-bit half-word (d mod 8) of the 128-bit Philox-4x32-10 output for
  counter (floor(d / 8), v mod 2^32, floor(v / 2^32), 0) and key (seed mod 2^32,
  floor(seed / 2^32)): words in order, the low half first. A value never depends on the
  vocabulary chunking or on the launch that computes it.
* A zero result is stored as +0.

The grid neighbours are found by searching the sorted table of every finite value of the
format, the plain definition.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16, decode_fp8_e4m3fn, encode_fp8_e4m3fn
from .philox import philox4x32

FP8_MAX = 448.0


def uniform16(v, d, seed: int) -> np.ndarray:
    """u in [0, 1), multiples of 2^-16, for elements (v, d) (broadcast int arrays)."""
    v = np.asarray(v, dtype=np.uint64)
    d = np.asarray(d, dtype=np.uint64)
    v, d = np.broadcast_arrays(v, d)
    ctr = np.stack([d >> np.uint64(3), v & np.uint64(0xFFFFFFFF), v >> np.uint64(32), np.zeros_like(v)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32(ctr, key).astype(np.uint64)
    j = (d & np.uint64(7)).astype(np.int64)
    w = np.take_along_axis(words, (j >> 1)[..., None], axis=-1)[..., 0]
    h = np.where((j & 1) == 1, w >> np.uint64(16), w & np.uint64(0xFFFF))
    return h.astype(np.float64) / 65536.0


def _grid(fmt: str) -> np.ndarray:
    if fmt == "fp8":
        vals = decode_fp8_e4m3fn(np.arange(256, dtype=np.uint8))
    elif fmt == "bf16":
        vals = decode_bf16(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    else:
        raise ValueError(fmt)
    return np.unique(vals[np.isfinite(vals)])


def sr_round(y, u, fmt: str) -> np.ndarray:
    """Stochastic rounding of y (float64) with uniforms u onto the fmt grid; float64 values."""
    g = _grid(fmt)
    y = np.asarray(y, dtype=np.float64)
    if fmt == "fp8":
        y = np.clip(y, -FP8_MAX, FP8_MAX)
    if np.any(y < g[0]) or np.any(y > g[-1]):
        raise ValueError("value outside the format's finite range")
    hi = g[np.searchsorted(g, y, side="left")]
    lo = g[np.searchsorted(g, y, side="right") - 1]
    out = np.where(lo == hi, y, np.where(np.asarray(u) * (hi - lo) < y - lo, hi, lo))
    return out + 0.0                                   # -0 -> +0


def encode(vals, fmt: str) -> np.ndarray:
    """Grid values to storage codes (exact)."""
    vals = np.asarray(vals, dtype=np.float64)
    if fmt == "fp8":
        return encode_fp8_e4m3fn(vals)
    bits = vals.astype(np.float32).view(np.uint32)
    return (bits >> 16).astype(np.uint16)


def decode(codes, fmt: str) -> np.ndarray:
    return decode_fp8_e4m3fn(codes) if fmt == "fp8" else decode_bf16(codes)


def sgd_sr(E_codes, items, dE, lr: float, seed: int, fmt: str) -> np.ndarray:
    """E' codes of the given item rows: SR(E - lr dE) with the (v, d)-keyed uniforms.
    E_codes [R, D] (the rows of `items`), dE [R, D] float64."""
    E = decode(E_codes, fmt)
    R, D = E.shape
    u = uniform16(np.asarray(items, dtype=np.int64)[:, None], np.arange(D)[None, :], seed)
    y = E - lr * np.asarray(dE, dtype=np.float64)
    return encode(sr_round(y, u, fmt), fmt)
