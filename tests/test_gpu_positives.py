"""The sparse correction's positive logits on their own scale (Cut Binary Cross Entropy,
§I-B, fused direct BCE formulation: loss_t = sum_v softplus(x_tv) - sum_p x_tp).

At full vocabulary size the positive-logit sum is a tiny part of the loss, so the loss
tolerance says nothing about it. These tests read the positive logits the loss uses
(cutloss_bce_positive_logits) and compare every canonical pair and every row sum with the
oracle's fp64 indexed dot products:
  * each x_tp within the fp32 evaluation band of its dot product (oracle.metrics
    decision_band, pinned on the CPU against fp32 evaluations in several orders), and
    within 1e-3 of |x_tp| wherever |x_tp| exceeds that band by 1000x;
  * each row sum within 1e-3 of sum_p |x_tp| plus the sum of the terms' bands.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from oracle.metrics import decision_band
from workloads import make, workload
from workloads.gen import Workload

from gpu_util import canonical, decode_inputs, dev, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def _say(msg):
    print(f"[positives] {msg}", flush=True)


def _pair_band(A, E, crow, cids, D):
    rows = np.repeat(np.arange(A.shape[0]), np.diff(crow))
    band = np.empty(len(cids))
    step = 65536
    for i in range(0, len(cids), step):   # the band of each pair's own dot product
        r, c = rows[i:i + step], cids[i:i + step]
        band[i:i + step] = (D * 2.0 ** -23) * np.einsum("ij,ij->i", np.abs(A[r]), np.abs(E[c]))
    return band


def _check(B, inp, pad_id):
    w = inp["workload"]
    g = upload(inp)
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], pad_id)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_FWD), g["A"].device)
    sum_x = torch.full((w.T,), float("nan"), dtype=torch.float32, device=dev())
    nnz = len(inp["ids"])
    x_pos = torch.full((max(nnz, 1),), float("nan"), dtype=torch.float32, device=dev())
    B.cutloss_bce_positive_logits(prob, sum_x, x_pos, ws)
    torch.cuda.synchronize()
    A64, E64 = decode_inputs(inp)
    crow, cids, n_bad = canonical(inp, w.V, pad_id)
    assert B.cutloss_read_data_errors(ws) == n_bad
    xr, sr = H.positive_logits(A64, E64, crow, cids)
    n = len(cids)
    xg = x_pos.cpu().numpy().astype(np.float64)[:n]
    sg = sum_x.cpu().numpy().astype(np.float64)
    band = _pair_band(A64, E64, crow, cids, w.D)
    # a spot check that the band is the right formula for these pairs
    if n:
        k = min(n - 1, 7)
        t = int(np.searchsorted(crow, k, side="right") - 1)
        assert band[k] == pytest.approx(decision_band(A64[t:t + 1], E64[cids[k]:cids[k] + 1], w.D)[0, 0], rel=1e-12)
    err = np.abs(xg - xr)
    bad = np.nonzero(err > band)[0]
    assert len(bad) == 0, f"x_tp outside the fp32 band at pairs {bad[:5]}: got {xg[bad[:5]]} ref {xr[bad[:5]]}"
    big = np.abs(xr) > 1000 * band
    assert np.all(err[big] <= 1e-3 * np.abs(xr[big]))
    rows = np.repeat(np.arange(w.T), np.diff(crow))
    mag = np.bincount(rows, weights=np.abs(xr), minlength=w.T)
    row_band = np.bincount(rows, weights=band, minlength=w.T)
    serr = np.abs(sg - sr)
    bad = np.nonzero(serr > 1e-3 * mag + row_band)[0]
    assert len(bad) == 0, f"row sums out of tolerance at rows {bad[:5]}: got {sg[bad[:5]]} ref {sr[bad[:5]]}"
    empty = np.diff(crow) == 0
    assert np.all(sg[empty] == 0)
    rel = float(np.max(serr / np.maximum(mag, 1e-30))) if n else 0.0
    _say(f"{w.name}: {n} pairs, max |err| {err.max() if n else 0:.3e}, "
         f"max row err / sum|x| {rel:.3e}, max err / band {float(np.max(err / band)) if n else 0:.3f}")


@pytest.mark.parametrize("D,e_dtype", [(128, "bf16"), (384, "bf16"), (768, "fp8")])
def test_positive_logits_small(B, D, e_dtype):
    """Pads, repeats, masked rows, empty rows, out-of-range IDs (counted, dropped)."""
    _say(f"small D={D} {e_dtype}")
    w = Workload("pos_small", "bce", 300, D, 5000, e_dtype, None, None, "uniform_any", L=12, pad_id=0,
                 mask_frac=0.2, seed=21)
    inp = make(w)
    ids = inp["ids"].copy()
    ids[::53] = w.V + 3
    inp["ids"] = ids
    rp = inp["row_ptr"].copy()     # row 5 without IDs
    n5 = rp[6] - rp[5]
    inp["ids"] = np.delete(ids, np.arange(rp[5], rp[6]))
    rp[6:] -= n5
    inp["row_ptr"] = rp
    _check(B, inp, 0)


@pytest.mark.parametrize("name", ["seqrec_bce", "xmc_sgd", "seqrec_bce_large"])
def test_positive_logits_full_size(B, name):
    """Every canonical pair of the full-size heads (the sequential-recommendation heads at
    V=876,939 with D=256 and D=512, the XMC head at V=3,000,000 with FP8 E)."""
    _say(f"full size {name}")
    _check(B, make(workload(name)), 0)
