"""GPU parity of the chunked path (heads with D outside {64, 128, 256}, or FP8 E)
against the fp64 CPU oracle, with the chunk size capped so that every case spans
several vocabulary chunks and a ragged last chunk (CUTLOSS_MAX_CHUNK_ITEMS).
Tolerances are those of tests/gpu_util.py.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from workloads import make
from workloads.gen import Workload

from gpu_util import (bf16_to_f64, canonical, check_grad, check_loss, decode_inputs, run_bce, run_ce, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


@pytest.fixture(autouse=True)
def small_chunks(monkeypatch):
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "512")


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _bce_check(B, inp, pad_id, dloss=None):
    w = inp["workload"]
    A64, E64 = decode_inputs(inp)
    crow, cids, n_bad = canonical(inp, w.V, pad_id)
    g = upload(inp)
    dl = None if dloss is None else torch.from_numpy(dloss).to(g["A"].device)
    out = run_bce(B, g, pad_id, dloss=dl)
    ref_loss = H.bce_loss(A64, E64, crow, cids, inp["mask"])
    check_loss(out["loss"].cpu().numpy(), ref_loss, what="fwd loss")
    check_loss(out["floss"].cpu().numpy(), ref_loss, what="fused loss")
    assert out["n_err"] == n_bad
    dA, dE = H.bce_grads(A64, E64, crow, cids, inp["mask"], dloss)
    check_grad(bf16_to_f64(out["dA"]), dA, "dA")
    check_grad(bf16_to_f64(out["dE"]), dE, "dE")
    m = inp["mask"] == 0
    if m.any():
        assert np.all(out["loss"].cpu().numpy()[m] == 0)
        assert np.all(bf16_to_f64(out["dA"])[m] == 0)
    return out


# D = 1088 (above 1024, at most 128 rows): 8-wave logits workgroups whose four wave rows merge
# their loss partials per item tile
@pytest.mark.parametrize("T,D,V", [(70, 320, 3001), (129, 512, 1001), (33, 768, 700), (300, 384, 2100), (40, 1088, 900)])
def test_bce_chunked_ragged(B, T, D, V):
    _say(f"chunked bce T={T} D={D} V={V}")
    w = Workload("chunk", "bce", T, D, V, "bf16", None, None, "uniform_any", L=10, pad_id=0, mask_frac=0.15,
                 seed=200 + T)
    inp = make(w, with_dloss=True)
    _bce_check(B, inp, 0, dloss=inp["dloss"])


def test_bce_chunked_stress_scale(B):
    # A, E ~ N(0, I) as in the Cut BCE mini-benchmark (§IV-A): saturated sigmoids
    _say("chunked bce stress N(0,1) T=64 D=384 V=1500")
    w = Workload("chunk_stress", "bce", 64, 384, 1500, "bf16", 1.0, 1.0, "uniform_any", L=8, pad_id=0, seed=21)
    _bce_check(B, make(w), 0)


def test_bce_chunked_closed_forms(B):
    w = Workload("chunk_cf", "bce", 50, 384, 1300, "bf16", None, None, "uniform_any", L=6, pad_id=0, mask_frac=0.1,
                 seed=22)
    inp = make(w)
    for zero in ("A", "E"):
        _say(f"chunked closed form {zero}=0")
        z = dict(inp)
        z[zero] = np.zeros_like(inp[zero])
        out = _bce_check(B, z, 0)
        valid = z["mask"] != 0
        np.testing.assert_allclose(out["loss"].cpu().numpy()[valid], w.V * math.log(2.0), rtol=1e-5)


def _sgd_case(B, T, D, V, seed):
    w = Workload("sgd", "bce", T, D, V, "fp8", None, 0.05, "poisson_distinct", L=5, pad_id=-1, lr=0.01, seed=seed)
    inp = make(w)
    A64, E64 = decode_inputs(inp)
    crow, cids, _ = canonical(inp, w.V, -1)
    g = upload(inp)
    dev = g["A"].device
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], -1)
    # one workspace for the unfused backward and the SGD step: large enough for both
    ws = B.workspace(max(B.cutloss_bce_workspace_size(prob, B.OP_FWD), B.cutloss_bce_workspace_size(prob, B.OP_BWD),
                         B.cutloss_bce_workspace_size(prob, B.OP_BWD_SGD)), dev)
    # the forward alone (for T <= 128 and D <= 768 the streaming logits product's loss-only mode)
    lossf = torch.empty(w.T, dtype=torch.float32, device=dev)
    B.cutloss_bce_fwd(prob, lossf, ws)
    dE = torch.empty(w.V, w.D, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev)
    B.cutloss_bce_bwd(prob, None, dA, dE, None, ws)
    loss = torch.empty(w.T, dtype=torch.float32, device=dev)
    dA2 = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev)
    B.cutloss_bce_bwd_sgd(prob, None, w.lr, dA2, loss, ws)
    torch.cuda.synchronize()
    dA_ref, dE_ref = H.bce_grads(A64, E64, crow, cids, inp["mask"])
    check_grad(bf16_to_f64(dE), dE_ref, "dE (fp8 E)")
    check_grad(bf16_to_f64(dA), dA_ref, "dA (fp8 E)")
    # the fused call reads E before updating it: its dA and loss are those of the old E
    check_grad(bf16_to_f64(dA2), dA_ref, "dA (fused SGD call)")
    loss_ref = H.bce_loss(A64, E64, crow, cids, inp["mask"])
    check_loss(lossf.cpu().numpy(), loss_ref, what="forward loss")
    check_loss(loss.cpu().numpy(), loss_ref, what="sgd fused loss")
    from test_gpu_parity import _check_sgd
    _check_sgd(g["E"].cpu().numpy(), inp["E"], dE_ref, w.lr)


def test_sgd_fp8_chunked_wide(B):
    _say("chunked fp8 SGD T=40 D=768 V=2000")
    _sgd_case(B, 40, 768, 2000, 31)


def test_sgd_fp8_chunked_ragged(B):
    _say("chunked fp8 SGD T=130 D=192 V=1537")
    _sgd_case(B, 130, 192, 1537, 32)


@pytest.mark.parametrize("T,D,V", [(1, 128, 33), (128, 1024, 700), (97, 896, 1000), (64, 256, 1000),
                                   (128, 384, 517), (100, 512, 2049), (7, 640, 300)])
def test_sgd_fp8_whole_rows(B, T, D, V):
    """The nearest-even FP8 SGD of heads of at most 128 rows updates whole E rows: one row,
    a 32-item block that ends a row past the vocabulary, eight and seven 128-column slices,
    and two to five slices; at D <= 768 the logits come from the streaming logits product
    (each of its head widths: loss-only forward, loss and gradient tile for the backward)."""
    _say(f"fp8 SGD whole rows T={T} D={D} V={V}")
    _sgd_case(B, T, D, V, 40 + T)


@pytest.mark.parametrize("T,D,V", [(70, 384, 3001), (33, 2304, 700), (257, 512, 1300)])
def test_ce_chunked(B, T, D, V):
    _say(f"chunked ce T={T} D={D} V={V}")
    w = Workload("ce_chunk", "ce", T, D, V, "bf16", None, None, "ce_uniform", L=1, pad_id=-1, ignore_frac=0.1,
                 seed=300 + T)
    inp = make(w, with_dloss=True)
    tgt = inp["target"].copy()
    tgt[1] = V + 7          # out of range: counted, row ignored
    inp["target"] = tgt
    g = upload(inp)
    A64, E64 = decode_inputs(inp)
    out = run_ce(B, g, dloss=g["dloss"])
    loss, lse = H.ce_forward(A64, E64, tgt)
    check_loss(out["lse"].cpu().numpy(), lse, what="lse")
    check_loss(out["loss"].cpu().numpy(), loss, what="loss")
    dA, dE = H.ce_grads(A64, E64, tgt, dloss=inp["dloss"])
    check_grad(bf16_to_f64(out["dA"]), dA, "dA")
    check_grad(bf16_to_f64(out["dE"]), dE, "dE")
    assert out["n_err"] == 1


def test_chunked_determinism_reused_workspace(B):
    """Two calls on one reused workspace give identical bits on the chunked path: split-K dA
    partials, their fixed-order reduction, the loss partials and the dE product (BCE at
    D = 512 over six 512-item chunks), and the CE path with and without the gradient filter."""
    _say("chunked determinism, reused workspace")
    w = Workload("det_chunk", "bce", 300, 512, 2900, "bf16", None, None, "zipf", L=8, pad_id=0, mask_frac=0.1,
                 seed=23)
    g = upload(make(w))
    dev = g["A"].device
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], 0)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD), dev)
    outs = []
    for _ in range(2):
        loss = torch.empty(w.T, dtype=torch.float32, device=dev)
        dA = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev)
        dE = torch.empty(w.V, w.D, dtype=torch.bfloat16, device=dev)
        B.cutloss_bce_bwd(prob, None, dA, dE, loss, ws)
        outs.append((loss, dA.view(torch.int16), dE.view(torch.int16)))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)

    wc = Workload("det_ce", "ce", 257, 384, 2100, "bf16", 1.0, 1.0, "ce_uniform", L=1, pad_id=-1, ignore_frac=0.1,
                  seed=24)
    gc = upload(make(wc))
    pc = B.ce_problem(gc["A"], gc["E"], gc["target"], -100)
    wsc = B.workspace(max(B.cutloss_ce_workspace_size(pc, B.OP_BWD), B.cutloss_ce_workspace_size(pc, B.OP_FWD)), dev)
    for eps in (None, 2.0 ** -12):
        res = []
        for _ in range(2):
            loss = torch.empty(wc.T, dtype=torch.float32, device=dev)
            lse = torch.empty(wc.T, dtype=torch.float32, device=dev)
            B.cutloss_ce_fwd(pc, loss, lse, wsc)
            dA = torch.empty(wc.T, wc.D, dtype=torch.bfloat16, device=dev)
            dE = torch.empty(wc.V, wc.D, dtype=torch.bfloat16, device=dev)
            if eps is None:
                B.cutloss_ce_bwd(pc, lse, None, dA, dE, wsc)
            else:
                B.cutloss_ce_bwd_filtered(pc, lse, None, dA, dE, eps, wsc)
            res.append((loss, lse, dA.view(torch.int16), dE.view(torch.int16)))
        torch.cuda.synchronize()
        for a, b in zip(*res):
            assert torch.equal(a, b), f"CE eps={eps}"
