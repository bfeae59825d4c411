"""Cut Metrics, plain definition (oracle; test infrastructure: only the tests, smoke() and
the bench's CPU baseline use it).

Cut Binary Cross Entropy (paperpeel), §III-D "Zero-Overhead Cut Metrics": per row of the
[B, N] grid the TP, FP, FN and TN counts over the item vocabulary, computed during the
forward pass without forming the logits. Here the counts are written out over the
materialized logits X = A E^T.

Reading (the section states no threshold): a prediction is positive when sigmoid(x) > 0.5,
that is x > 0, the usual default threshold of binary-classification metrics. Labels are the
canonical positive sets (pads dropped, repeats once). Masked rows give (0, 0, 0, 0).

Floating point decides these integers. ``decision_band`` bounds the fp32 rounding of a
logit computed from the same bf16/fp8 operands in any summation order, and
``cut_metrics_rows`` reports the counts with each logit inside that band taken either way,
so that a check can accept exactly the decisions a correct fp32 evaluation can make.
"""
from __future__ import annotations

import numpy as np


def _valid_rows(T: int, mask) -> np.ndarray:
    return np.ones(T, dtype=bool) if mask is None else np.asarray(mask) != 0


def cut_metrics(A, E, crow, cids, mask=None) -> np.ndarray:
    """counts[t] = (TP, FP, FN, TN) of the predictions x_tv > 0 against P_t, int64 [T, 4]."""
    T, V = A.shape[0], E.shape[0]
    X = A @ E.T
    valid = _valid_rows(T, mask)
    out = np.zeros((T, 4), dtype=np.int64)
    for t in range(T):
        if not valid[t]:
            continue
        y = np.zeros(V, dtype=bool)
        y[cids[crow[t]:crow[t + 1]]] = True
        pred = X[t] > 0.0
        tp = int(np.sum(pred & y))
        fp = int(np.sum(pred & ~y))
        fn = int(np.sum(~pred & y))
        tn = int(np.sum(~pred & ~y))
        out[t] = (tp, fp, fn, tn)
    return out


def decision_band(A_rows, E, D: int) -> np.ndarray:
    """|fp32 evaluation - exact value| bound for every logit of the given rows: D * 2^-23 *
    sum_d |a_d e_d| (a generous form of the gamma_D bound of a length-D fp32 dot product)."""
    return (D * 2.0 ** -23) * (np.abs(A_rows) @ np.abs(E).T)


def cut_metrics_rows(A, E, crow, cids, rows, mask=None):
    """For each sampled row: the exact counts, and the interval of TP and of the number of
    predicted positives that a correct fp32 evaluation can produce.

    Returns (counts [R, 4], tp_lo, tp_hi, pos_lo, pos_hi), all int64 arrays of length R
    (counts 2-D). Masked rows have all of them 0."""
    T, V, D = A.shape[0], E.shape[0], A.shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    X = A[rows] @ E.T
    band = decision_band(A[rows], E, D)
    valid = _valid_rows(T, mask)[rows]
    R = len(rows)
    counts = np.zeros((R, 4), dtype=np.int64)
    tp_lo = np.zeros(R, dtype=np.int64)
    tp_hi = np.zeros(R, dtype=np.int64)
    pos_lo = np.zeros(R, dtype=np.int64)
    pos_hi = np.zeros(R, dtype=np.int64)
    for i, t in enumerate(rows):
        if not valid[i]:
            continue
        y = np.zeros(V, dtype=bool)
        y[cids[crow[t]:crow[t + 1]]] = True
        x, b = X[i], band[i]
        pred = x > 0.0
        surely = x > b          # positive under any correct fp32 evaluation
        maybe = x > -b          # positive under some correct fp32 evaluation
        tp = int(np.sum(pred & y))
        fp = int(np.sum(pred & ~y))
        npos = int(y.sum())
        counts[i] = (tp, fp, npos - tp, V - npos - fp)
        tp_lo[i], tp_hi[i] = int(np.sum(surely & y)), int(np.sum(maybe & y))
        pos_lo[i], pos_hi[i] = int(np.sum(surely)), int(np.sum(maybe))
    return counts, tp_lo, tp_hi, pos_lo, pos_hi
