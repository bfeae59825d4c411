"""Canonical positive sets of the multi-label targets (oracle's own code).

Cut Binary Cross Entropy (paperpeel): §III-B keeps only the sparse [B,N,L]
target IDs (no multi-hot tensor); §III-E trains every non-padding position and
pads target lists; §IV-A tests padded and duplicate target IDs. Read together:
the label y_tv of row t and item v is 1 exactly when v appears in row t's list,
is not the padding ID, and row t is valid. Repeats count once (y is 0/1).

Readings where the pages are silent:
* an ID outside [0, V) that is not the padding ID is a data error: it is
  counted (each occurrence, valid rows only) and otherwise ignored;
* a masked row has an empty set (and, in the loss, weight 0).
"""
from __future__ import annotations

import numpy as np


def canonical_sets(row_ptr, ids, mask, V: int, pad_id: int):
    """Per row, the sorted distinct positive item IDs; plus the count of bad IDs."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    T = len(row_ptr) - 1
    mask = np.ones(T, dtype=np.uint8) if mask is None else np.asarray(mask, dtype=np.uint8)
    sets = []
    n_bad = 0
    for t in range(T):
        if not mask[t]:
            sets.append(np.zeros(0, dtype=np.int64))
            continue
        row = ids[row_ptr[t]:row_ptr[t + 1]]
        keep = []
        for v in row.tolist():
            if pad_id >= 0 and v == pad_id:
                continue
            if v < 0 or v >= V:
                n_bad += 1
                continue
            keep.append(v)
        sets.append(np.array(sorted(set(keep)), dtype=np.int64))
    return sets, n_bad


def canonical_csr(row_ptr, ids, mask, V: int, pad_id: int):
    """Canonical sets as CSR (row_ptr int64 [T+1], ids int64 [nnz']) and the bad-ID count."""
    sets, n_bad = canonical_sets(row_ptr, ids, mask, V, pad_id)
    crow = np.zeros(len(sets) + 1, dtype=np.int64)
    crow[1:] = np.cumsum([len(s) for s in sets])
    cids = np.concatenate(sets) if sets else np.zeros(0, dtype=np.int64)
    return crow, cids.astype(np.int64), n_bad


def item_major(crow, cids):
    """All (item, row) positive pairs, ordered by item then row."""
    T = len(crow) - 1
    rows = np.repeat(np.arange(T, dtype=np.int64), np.diff(crow))
    order = np.lexsort((rows, cids))
    return cids[order], rows[order]


def dense_labels(crow, cids, T: int, V: int) -> np.ndarray:
    """Multi-hot Y[T, V] in float64 (small shapes only)."""
    Y = np.zeros((T, V), dtype=np.float64)
    for t in range(T):
        Y[t, cids[crow[t]:crow[t + 1]]] = 1.0
    return Y
