"""GPU parity of the FP8-logits SGD step (cutloss_bce_bwd_sgd_ex with fp8_logits; ELMO,
ai.info summary, Methodology: activations cast to FP8 only for the matmul that produces the
logits) against the oracle's reading: X = fp8(A) E^T, loss and G from that X, dA = G E,
dE = G^T A with A itself. The logit product runs on the FP8 MFMA (64 k per instruction)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from oracle.formats import encode_fp8_e4m3fn
from oracle.stochastic import decode, sr_round, uniform16
from workloads import make, workload
from workloads.gen import Workload

from gpu_util import bf16_to_f64, canonical, check_grad, check_loss, decode_inputs, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _step(B, g, w, stochastic=False, seed=0, want_dA=True):
    dev = g["A"].device
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], w.pad_id)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD_SGD_EX), dev)
    loss = torch.empty(w.T, dtype=torch.float32, device=dev)
    dA = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev) if want_dA else None
    B.cutloss_bce_bwd_sgd_ex(prob, None, w.lr, dA, loss, ws, stochastic=stochastic, seed=seed, fp8_logits=True)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), (bf16_to_f64(dA) if want_dA else None)


def _check_E(E_new, E_old, items, dE_ref, lr, stochastic, seed):
    tol = 2e-2 * np.abs(dE_ref).max()
    y = decode(E_old, "fp8") - lr * dE_ref
    if stochastic:
        u = uniform16(np.asarray(items, dtype=np.int64)[:, None], np.arange(E_old.shape[1])[None, :], seed)
    else:
        u = None
    rnd = (lambda z: sr_round(z, u, "fp8")) if stochastic else (lambda z: decode(encode_fp8_e4m3fn(z), "fp8"))
    lo, hi, ex = rnd(y - lr * tol), rnd(y + lr * tol), rnd(y)
    got = decode(E_new, "fp8")
    assert np.all((got >= lo) & (got <= hi)), "E' outside the rounding interval"
    frac = float(np.mean(got != ex))
    print(f"[fp8 logits] E' differing from the rounding of E - lr dE_ref: {frac:.2e}")
    assert frac < 1e-2


@pytest.mark.parametrize("T,D,V,stochastic", [(40, 128, 2000, False), (70, 768, 3001, False),
                                               (130, 256, 1500, True), (128, 768, 2600, True)])
def test_fp8_logits_small(B, T, D, V, stochastic, monkeypatch):
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "512")
    _say(f"fp8 logits T={T} D={D} V={V} stochastic={stochastic}")
    w = Workload("f8l", "bce", T, D, V, "fp8", None, 0.05, "poisson_distinct", L=5, pad_id=-1, lr=0.01,
                 mask_frac=0.1, seed=31 + D + T)
    inp = make(w)
    A64, E64 = decode_inputs(inp)
    A8 = H.fp8_activations(A64)
    crow, cids, _ = canonical(inp, V, -1)
    g = upload(inp)
    loss, dA = _step(B, g, w, stochastic, seed=77)
    check_loss(loss, H.bce_loss(A64, E64, crow, cids, inp["mask"], A_logits=A8), what="fp8-logits loss")
    dA_ref, dE_ref = H.bce_grads(A64, E64, crow, cids, inp["mask"], A_logits=A8)
    check_grad(dA, dA_ref, "dA (fp8 logits)")
    _check_E(g["E"].cpu().numpy(), inp["E"], np.arange(V), dE_ref, w.lr, stochastic, 77)


def test_fp8_logits_follow_the_cast(B, monkeypatch):
    # the loss moves with the cast of A by far more than the GPU's own rounding: the GPU loss
    # must sit on the cast side, at under a tenth of the gap between the two readings
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "512")
    _say("fp8 vs bf16 logits T=64 D=64 V=1000")
    w = Workload("f8x", "bce", 64, 64, 1000, "fp8", 1.0, 0.05, "poisson_distinct", L=5, pad_id=-1, lr=0.01, seed=9)
    inp = make(w)
    A64, E64 = decode_inputs(inp)
    A8 = H.fp8_activations(A64)
    crow, cids, _ = canonical(inp, w.V, -1)
    ref8 = H.bce_loss(A64, E64, crow, cids, inp["mask"], A_logits=A8)
    ref16 = H.bce_loss(A64, E64, crow, cids, inp["mask"])
    gap = np.abs(ref8 - ref16)
    loss8, _ = _step(B, upload(inp), w, want_dA=False)
    check_loss(loss8, ref8, what="fp8-logits loss")
    valid = inp["mask"] != 0
    print(f"[fp8 logits] mean |gpu - fp8 reading| {np.mean(np.abs(loss8 - ref8)[valid]):.2e}, "
          f"mean gap to the bf16 reading {np.mean(gap[valid]):.2e}")
    assert np.mean(np.abs(loss8 - ref8)[valid]) < 0.1 * np.mean(gap[valid])


def test_fp8_logits_xmc_full_size_sampled(B):
    inp = make(workload("xmc_sgd"))
    w = inp["workload"]
    _say(f"fp8 logits full size T={w.T} D={w.D} V={w.V}")
    A64, E64 = decode_inputs(inp)
    A8 = H.fp8_activations(A64)
    crow, cids, _ = canonical(inp, w.V, w.pad_id)
    g = upload(inp)
    loss, dA = _step(B, g, w, stochastic=True, seed=5)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 32, replace=False)]))
    l_ref, dA_ref = H.bce_rows(A64, E64, crow, cids, rows, inp["mask"], A_logits=A8)
    check_loss(loss[rows], l_ref, what="fp8-logits loss (sampled rows)")
    check_grad(dA[rows], dA_ref, "dA (fp8 logits, sampled rows)")
    items = np.unique(np.concatenate([[0, 1, w.V - 1], np.unique(cids)[:32], rng.choice(w.V, 96, replace=False)]))
    dE_ref = H.bce_items(A64, E64, crow, cids, items, inp["mask"], A_logits=A8)
    E_new = g["E"][torch.from_numpy(items).to(g["E"].device)].cpu().numpy()
    _check_E(E_new, inp["E"][items], items, dE_ref, w.lr, True, 5)
