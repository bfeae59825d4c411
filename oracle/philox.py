"""Philox-4x32-10 counter-based generator (oracle; test infrastructure).

Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011),
the Philox-4x32 construction with 10 rounds. A 128-bit counter (four 32-bit words) and a
64-bit key (two words) map to 128 output bits. One round multiplies counter words 0 and
2 by the two Philox multipliers, keeps the 64-bit products' high and low halves, and
mixes the high halves with words 1 and 3 and the key:

    (hi0, lo0) = M0 * c0,   (hi1, lo1) = M1 * c2
    c' = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)

The key is incremented by the Weyl constants (W0, W1) between rounds (round r uses
k + (r - 1) W, modulo 2^32 per word).

The stochastic rounding of the SGD writeback draws from this generator; the kernels carry
their own implementation of the same published function.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
ROUNDS = 10
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32(counter, key, rounds: int = ROUNDS) -> np.ndarray:
    """counter: uint [..., 4]; key: uint [..., 2] (broadcast). Returns uint32 [..., 4]."""
    c = np.asarray(counter, dtype=np.uint64) & _MASK
    k = np.asarray(key, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = np.uint64(M0) * c0            # < 2^64: exact in uint64
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)
