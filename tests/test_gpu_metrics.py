"""GPU parity of Cut Metrics (cutloss_bce_fwd_metrics; Cut Binary Cross Entropy, paperpeel,
§III-D) against the oracle's counts, on both paths.

Floating point decides the counts (x > 0). The oracle gives, per row, the interval of TP
and of the predicted-positive count that a correct fp32 evaluation of the same bf16/fp8
operands can produce (logits inside the rounding band go either way); the GPU counts must
lie inside it, FN and TN must follow exactly from TP and FP, and masked rows give zeros.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from oracle.metrics import cut_metrics_rows
from workloads import make, workload
from workloads.gen import Workload

from gpu_util import canonical, check_loss, decode_inputs, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _run(B, g, pad_id):
    A = g["A"]
    T = A.shape[0]
    prob = B.bce_problem(A, g["E"], g["row_ptr"], g["ids"], g.get("mask"), pad_id)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_FWD_METRICS), A.device)
    loss = torch.empty(T, dtype=torch.float32, device=A.device)
    counts = torch.empty(T, 4, dtype=torch.int32, device=A.device)
    B.cutloss_bce_fwd_metrics(prob, loss, counts, ws)
    ws2 = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_FWD), A.device)
    loss_plain = torch.empty(T, dtype=torch.float32, device=A.device)
    B.cutloss_bce_fwd(prob, loss_plain, ws2)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), counts.cpu().numpy().astype(np.int64), loss_plain.cpu().numpy()


def _check_counts(got, inp, crow, cids, rows, A64, E64):
    w = inp["workload"]
    _, tp_lo, tp_hi, pos_lo, pos_hi = cut_metrics_rows(A64, E64, crow, cids, rows, inp["mask"])
    mask = inp["mask"]
    amb = 0
    for i, t in enumerate(rows):
        tp, fp, fn, tn = got[i]
        if mask[t] == 0:
            assert (tp, fp, fn, tn) == (0, 0, 0, 0), f"row {t}: masked row counts {got[i]}"
            continue
        npos = crow[t + 1] - crow[t]
        assert tp_lo[i] <= tp <= tp_hi[i], f"row {t}: TP {tp} outside [{tp_lo[i]}, {tp_hi[i]}]"
        assert fp >= 0 and fn == npos - tp and tn == w.V - npos - fp, f"row {t}: counts {got[i]}"
        # FP = predicted positives - TP, each decided inside its band
        assert pos_lo[i] - tp_hi[i] <= fp <= pos_hi[i] - tp_lo[i], f"row {t}: FP {fp}"
        amb += (tp_hi[i] - tp_lo[i]) + (pos_hi[i] - pos_lo[i])
    print(f"[metrics] rows {len(rows)}, logits inside the rounding band: {amb}")


@pytest.mark.parametrize("T,D,V,e", [(70, 64, 3001, "bf16"), (129, 128, 1001, "bf16"), (200, 256, 4097, "bf16"),
                                     (90, 384, 2100, "bf16"), (64, 256, 1500, "fp8"), (40, 1088, 900, "bf16"),
                                     (100, 640, 1700, "fp8"), (128, 768, 3000, "fp8")])
def test_metrics_small(B, T, D, V, e, monkeypatch):
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "512")
    _say(f"metrics T={T} D={D} V={V} E {e}")
    # A, E ~ N(0, 1): many logits far from 0 and a spread of signs
    w = Workload("metrics", "bce", T, D, V, e, 1.0, 1.0, "uniform_any", L=9, pad_id=0, mask_frac=0.15, seed=400 + T)
    inp = make(w)
    A64, E64 = decode_inputs(inp)
    crow, cids, _ = canonical(inp, V, 0)
    loss, counts, loss_plain = _run(B, upload(inp), 0)
    assert np.array_equal(loss, loss_plain), "the metrics forward changed the loss"
    check_loss(loss, H.bce_loss(A64, E64, crow, cids, inp["mask"]), what="loss (metrics forward)")
    rows = np.arange(T)
    _check_counts(counts, inp, crow, cids, rows, A64, E64)


def test_metrics_closed_form(B):
    # A_t = u, E_v = +u on a set S and -u elsewhere: x = +-1 up to rounding, counts exact
    _say("metrics closed form")
    T, D, V = 3, 64, 700
    u = np.full(D, 0.125, dtype=np.float32)              # sum u^2 = 1, exact in bf16
    S = np.array([0, 5, 77, 300, 699])
    E = -np.tile(u, (V, 1))
    E[S] = u
    A = np.tile(u, (T, 1))
    to_bf16 = lambda x: (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    row_ptr = np.array([0, 3, 4, 7], dtype=np.int32)
    ids = np.array([5, 6, 300, 699, 0, 1, 2], dtype=np.int32)
    inp = {"workload": Workload("cf", "bce", T, D, V, "bf16", None, None, "uniform_any", L=3, pad_id=-1),
           "A": to_bf16(A), "E": to_bf16(E), "row_ptr": row_ptr, "ids": ids, "mask": np.ones(T, dtype=np.uint8)}
    _, counts, _ = _run(B, upload(inp), -1)
    nS = len(S)
    assert tuple(counts[0]) == (2, nS - 2, 1, V - 3 - (nS - 2))    # P = {5, 6, 300}
    assert tuple(counts[1]) == (1, nS - 1, 0, V - 1 - (nS - 1))    # P = {699}
    assert tuple(counts[2]) == (1, nS - 1, 2, V - 3 - (nS - 1))    # P = {0, 1, 2}


def test_metrics_full_size_sampled(B):
    inp = make(workload("seqrec_bce"))
    w = inp["workload"]
    _say(f"metrics full size T={w.T} D={w.D} V={w.V}")
    A64, E64 = decode_inputs(inp)
    crow, cids, _ = canonical(inp, w.V, 0)
    loss, counts, loss_plain = _run(B, upload(inp), 0)
    assert np.array_equal(loss, loss_plain)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, w.T - 1], np.nonzero(inp["mask"] == 0)[0][:4],
                                     rng.choice(w.T, 64, replace=False)]))
    _check_counts(counts[rows], inp, crow, cids, rows, A64, E64)
