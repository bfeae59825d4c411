"""Pins of the Cut Metrics oracle (Cut Binary Cross Entropy, paperpeel, §III-D) against a
library routine, closed forms and identities, independent of the oracle's own code."""
from __future__ import annotations

import numpy as np
import pytest
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


# ---------------------------------------------------------------- the decision band itself

def _fp32_dots(p):
    """float32 sums of the exact float32 products p[..., D] in several orders: sequential,
    reversed, a pairwise tree, blocks of 16 and 32 summed in float32 and then across blocks
    (the k step of the bf16 matrix instructions), and a fixed random permutation."""
    p = np.asarray(p, dtype=np.float32)
    D = p.shape[-1]

    def seq(q):
        s = np.zeros(q.shape[:-1], dtype=np.float32)
        for k in range(q.shape[-1]):
            s = (s + q[..., k]).astype(np.float32)
        return s

    def tree(q):
        while q.shape[-1] > 1:
            if q.shape[-1] % 2:
                q = np.concatenate([q, np.zeros(q.shape[:-1] + (1,), np.float32)], axis=-1)
            q = (q[..., 0::2] + q[..., 1::2]).astype(np.float32)
        return q[..., 0]

    def blocks(q, b):
        parts = [seq(q[..., i:i + b]) for i in range(0, q.shape[-1], b)]
        return seq(np.stack(parts, axis=-1))

    perm = np.random.default_rng(0).permutation(D)
    return [seq(p), seq(p[..., ::-1]), tree(p), blocks(p, 16), blocks(p, 32), seq(p[..., perm])]


@pytest.mark.parametrize("D,std", [(64, None), (256, None), (768, None), (256, 1.0)])
def test_decision_band_covers_fp32_evaluations(D, std):
    """Every float32 evaluation order of a logit of bf16 operands lies within the band of
    the exact value (products of two bf16 values are exact in float32)."""
    import torch
    from oracle.formats import decode_bf16
    from oracle.metrics import decision_band
    rng = np.random.default_rng(D)
    s = std if std is not None else 1.0 / np.sqrt(D)

    def bf16(x):
        return decode_bf16(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
                           .view(np.uint16))
    A = bf16(rng.normal(0, s, (24, D)))
    E = bf16(rng.normal(0, s, (200, D)))
    exact = A @ E.T                                          # float64: error far below the band
    band = decision_band(A, E, D)
    prods = (A[:, None, :] * E[None, :, :]).astype(np.float32)
    assert np.array_equal(prods.astype(np.float64), A[:, None, :] * E[None, :, :])
    worst = 0.0
    for got in _fp32_dots(prods):
        err = np.abs(got.astype(np.float64) - exact)
        assert np.all(err <= band)
        worst = max(worst, float((err / band).max()))
    assert worst > 0.0


@pytest.mark.parametrize("D", [16, 64, 256, 1024])
def test_decision_band_is_within_a_small_factor_of_a_reachable_error(D):
    """A sequential float32 sum that loses every small term: a = (1, d, d, ...), e = 1 with
    d the largest bf16 value below half an ulp of 1. The float32 sum stays 1, an error of
    (D - 1) d, about half the band: a band without its factor D would not cover it, and
    one more than 4x wider than needed fails the second check."""
    from oracle.metrics import decision_band
    d = (1.0 - 2.0 ** -8) * 2.0 ** -24                     # 8 significant bits: a bf16 value
    a = np.full(D, d)
    a[0] = 1.0
    e = np.ones(D)
    got = _fp32_dots(a[None, None, :] * e)[0][0, 0]
    assert got == np.float32(1.0)
    err = abs(float(got) - (1.0 + (D - 1) * d))
    band = float(decision_band(a[None, :], e[None, :], D)[0, 0])
    assert err <= band
    assert err >= band / 4
