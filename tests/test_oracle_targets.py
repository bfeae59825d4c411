"""Pins of the oracle's canonical positive sets against hand-written cases."""
import json
import os

import numpy as np
import pytest

from oracle.targets import canonical_csr, canonical_sets, dense_labels, item_major

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "targets_cases.json")
CASES = json.load(open(GOLDEN))["cases"]


def _csr(rows):
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    ids = np.array([v for r in rows for v in r], dtype=np.int32)
    return row_ptr, ids


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_canonical_sets_golden(case):
    row_ptr, ids = _csr(case["rows"])
    sets, n_bad = canonical_sets(row_ptr, ids, np.array(case["mask"], np.uint8), case["V"], case["pad_id"])
    assert [s.tolist() for s in sets] == case["canonical"]
    assert n_bad == case["n_bad"]


def test_csr_and_item_major_order():
    row_ptr, ids = _csr([[4, 2, 2], [2, 9], [], [4, 0]])
    crow, cids, n_bad = canonical_csr(row_ptr, ids, None, 10, 0)
    assert crow.tolist() == [0, 2, 4, 4, 5] and cids.tolist() == [2, 4, 2, 9, 4] and n_bad == 0
    items, rows = item_major(crow, cids)
    assert items.tolist() == [2, 2, 4, 4, 9]
    assert rows.tolist() == [0, 1, 0, 3, 1]
    Y = dense_labels(crow, cids, 4, 10)
    assert Y.sum() == 5 and Y[3, 4] == 1 and Y[3, 0] == 0


def test_brute_force_random_lists():
    rng = np.random.default_rng(3)
    V, T = 50, 40
    rows = [rng.integers(-5, V + 5, size=rng.integers(0, 12)).tolist() for _ in range(T)]
    mask = (rng.random(T) > 0.2).astype(np.uint8)
    row_ptr, ids = _csr(rows)
    sets, n_bad = canonical_sets(row_ptr, ids, mask, V, 0)
    bad = 0
    for t in range(T):
        want = set()
        for v in rows[t]:
            if not mask[t] or v == 0:
                continue
            if 0 <= v < V:
                want.add(v)
            else:
                bad += 1
        assert sets[t].tolist() == sorted(want)
    assert n_bad == bad
