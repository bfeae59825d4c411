"""Pins of the Cut Metrics oracle (Cut Binary Cross Entropy, paperpeel, §III-D) against a
library routine, closed forms and identities, independent of the oracle's own code."""
from __future__ import annotations

import numpy as np
from sklearn.metrics import confusion_matrix

from oracle.metrics import cut_metrics, cut_metrics_rows
from oracle.targets import canonical_csr


def _problem(T, D, V, L, seed, mask_frac=0.0):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((T, D))
    E = rng.standard_normal((V, D))
    row_ptr = np.arange(0, T * L + 1, L, dtype=np.int32)
    ids = rng.integers(0, V, size=T * L).astype(np.int32)
    mask = np.ones(T, dtype=np.uint8)
    mask[rng.permutation(T)[:int(round(mask_frac * T))]] = 0
    crow, cids, _ = canonical_csr(row_ptr, ids, mask, V, -1)
    return A, E, crow, cids, mask


def test_matches_sklearn_confusion_matrix():
    A, E, crow, cids, mask = _problem(12, 8, 57, 5, seed=1, mask_frac=0.25)
    got = cut_metrics(A, E, crow, cids, mask)
    X = A @ E.T
    for t in range(A.shape[0]):
        if mask[t] == 0:
            assert np.all(got[t] == 0)
            continue
        y = np.zeros(E.shape[0], dtype=int)
        y[cids[crow[t]:crow[t + 1]]] = 1
        tn, fp, fn, tp = confusion_matrix(y, (X[t] > 0).astype(int), labels=[0, 1]).ravel()
        assert tuple(got[t]) == (tp, fp, fn, tn)


def test_identities():
    A, E, crow, cids, mask = _problem(20, 16, 300, 7, seed=2, mask_frac=0.1)
    got = cut_metrics(A, E, crow, cids, mask)
    V = E.shape[0]
    for t in range(A.shape[0]):
        if mask[t] == 0:
            continue
        tp, fp, fn, tn = got[t]
        assert tp + fn == crow[t + 1] - crow[t]
        assert tp + fp + fn + tn == V
        assert tp + fp == int(np.sum(A[t] @ E.T > 0))


def test_closed_form_signed_items():
    # A_t = u and E_v = +u (v in S) or -u: x_tv > 0 exactly on S, for every row
    D, V = 8, 40
    u = np.ones(D) / np.sqrt(D)
    S = np.array([1, 4, 9, 16, 25, 36])
    E = -np.tile(u, (V, 1))
    E[S] = u
    A = np.tile(u, (3, 1))
    row_ptr = np.array([0, 3, 5, 9], dtype=np.int32)
    ids = np.array([1, 2, 3, 4, 5, 9, 16, 25, 36], dtype=np.int32)
    crow, cids, _ = canonical_csr(row_ptr, ids, None, V, -1)
    got = cut_metrics(A, E, crow, cids)
    # row 0: P = {1, 2, 3}: TP = {1}, FP = S - {1}, FN = {2, 3}
    assert tuple(got[0]) == (1, 5, 2, V - 8)
    # row 1: P = {4, 5}: TP = {4}, FP = 5, FN = {5}
    assert tuple(got[1]) == (1, 5, 1, V - 7)
    # row 2: P = {9, 16, 25, 36} subset of S: TP = 4, FP = 2, FN = 0
    assert tuple(got[2]) == (4, 2, 0, V - 6)


def test_zero_activations_predict_nothing():
    A, E, crow, cids, mask = _problem(6, 8, 50, 4, seed=3)
    got = cut_metrics(np.zeros_like(A), E, crow, cids, mask)
    for t in range(6):
        npos = crow[t + 1] - crow[t]
        assert tuple(got[t]) == (0, 0, npos, 50 - npos)


def test_sampled_rows_bracket_the_exact_counts():
    A, E, crow, cids, mask = _problem(16, 8, 120, 5, seed=4, mask_frac=0.2)
    full = cut_metrics(A, E, crow, cids, mask)
    rows = [0, 3, 7, 15]
    counts, tp_lo, tp_hi, pos_lo, pos_hi = cut_metrics_rows(A, E, crow, cids, rows, mask)
    assert np.array_equal(counts, full[rows])
    for i, t in enumerate(rows):
        assert tp_lo[i] <= full[t, 0] <= tp_hi[i]
        assert pos_lo[i] <= full[t, 0] + full[t, 1] <= pos_hi[i]
    # a logit at exactly 0 lies in its own band: both decisions are valid
    Az = np.zeros_like(A)
    _, tl, th, pl, ph = cut_metrics_rows(Az, E, crow, cids, [0], None)
    assert tl[0] == 0 and pl[0] == 0 and ph[0] == 0       # band 0 at A = 0: x = 0 is not > 0
