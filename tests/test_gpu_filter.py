"""GPU checks of the CE gradient filter (cutloss_ce_bwd_filtered; Cut Your Losses article,
the note on skipping the softmax tail below numerical precision), on both paths.

* eps = 0 reproduces cutloss_ce_bwd bit for bit.
* With eps > 0 the filtered gradient differs from the unfiltered one by no more than the
  oracle's bound on the dropped entries (all |w softmax| < eps), plus one bf16 rounding of
  each output. The bound carries a relative allowance of 2^-6: the unfiltered GPU result
  holds the dropped entries as bf16 softmax values (2^-9 each) from an fp32 exponential of
  an fp32 logit, and a column fed by a single row can reach the bound itself.
* With a near-uniform softmax over a large vocabulary every dense entry is below eps, so
  the result is the target-only gradient: dA_t = -w_t E_{y_t}, dE_v = -sum_{t: y_t = v} w_t A_t.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from workloads import make
from workloads.gen import Workload

from gpu_util import bf16_to_f64, decode_inputs, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _grads(B, g, eps=None, ws=None):
    A, E = g["A"], g["E"]
    T, D = A.shape
    V = E.shape[0]
    prob = B.ce_problem(A, E, g["target"], -100)
    if ws is None:
        ws = B.workspace(max(B.cutloss_ce_workspace_size(prob, B.OP_BWD), B.cutloss_ce_workspace_size(prob, B.OP_FWD)),
                         A.device)
    loss = torch.empty(T, dtype=torch.float32, device=A.device)
    lse = torch.empty(T, dtype=torch.float32, device=A.device)
    B.cutloss_ce_fwd(prob, loss, lse, ws)
    dA = torch.empty(T, D, dtype=torch.bfloat16, device=A.device)
    dE = torch.empty(V, D, dtype=torch.bfloat16, device=A.device)
    if eps is None:
        B.cutloss_ce_bwd(prob, lse, None, dA, dE, ws)
    else:
        B.cutloss_ce_bwd_filtered(prob, lse, None, dA, dE, eps, ws)
    torch.cuda.synchronize()
    return bf16_to_f64(dA), bf16_to_f64(dE)


BOUND_REL = 1.0 + 2.0 ** -6


def _check_moved(a0, a1, e0, e1, b_dA, b_dE):
    for name, x0, x1, b in (("dA", a0, a1, b_dA), ("dE", e0, e1, b_dE)):
        slack = 2.0 ** -8 * (np.abs(x0) + np.abs(x1))
        excess = np.abs(x1 - x0) - slack
        ratio = np.max(np.where(excess > 0, excess / (b + 1e-300), 0.0))
        print(f"[filter] {name}: largest move over the dropped-entry bound {ratio:.4f}")
        assert ratio <= BOUND_REL, f"{name} moved {ratio:.4f} x the dropped-entry bound"


def _case(T, D, V, scale, seed):
    w = Workload("filter", "ce", T, D, V, "bf16", scale, scale, "ce_uniform", L=1, pad_id=-1, ignore_frac=0.1,
                 seed=seed)
    return make(w)


@pytest.mark.parametrize("D", [64, 128, 256, 384])
def test_filter_off_is_exact(B, D, monkeypatch):
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "512")
    _say(f"filter eps=0, D={D}")
    g = upload(_case(70, D, 3001, 1.0, 600 + D))
    a0, e0 = _grads(B, g)
    a1, e1 = _grads(B, g, eps=0.0)
    assert np.array_equal(a0, a1) and np.array_equal(e0, e1)


@pytest.mark.parametrize("D", [64, 128, 256, 384])
def test_filter_within_dropped_bound(B, D, monkeypatch):
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "512")
    eps = 2.0 ** -12
    _say(f"filter eps=2^-12 peaked softmax, D={D}")
    inp = _case(96, D, 2600, 0.35, 700 + D)     # logits of std ~0.35^2 sqrt(D): a spread of tile maxima
    g = upload(inp)
    a0, e0 = _grads(B, g)
    a1, e1 = _grads(B, g, eps=eps)
    A64, E64 = decode_inputs(inp)
    b_dA, b_dE = H.ce_filter_bounds(A64, E64, inp["target"], eps)
    _check_moved(a0, a1, e0, e1, b_dA, b_dE)
    print(f"[filter] dA changed in {np.mean(a1 != a0):.3f} of elements, dE in {np.mean(e1 != e0):.3f}")


@pytest.mark.parametrize("D", [128, 384])
def test_filter_uniform_softmax_keeps_targets_only(B, D, monkeypatch):
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "1024")
    _say(f"filter uniform softmax, D={D}")
    inp = _case(64, D, 20000, 0.05, 800 + D)     # |x| << 1, softmax ~ 1/V = 5e-5 < 2^-12
    g = upload(inp)
    a1, e1 = _grads(B, g, eps=2.0 ** -12)
    A64, E64 = decode_inputs(inp)
    tgt = inp["target"]
    valid = (tgt != -100) & (tgt >= 0) & (tgt < E64.shape[0])
    ref_a = np.zeros_like(A64)
    ref_e = np.zeros_like(E64)
    for t in np.nonzero(valid)[0]:
        ref_a[t] = -E64[tgt[t]]
        ref_e[tgt[t]] -= A64[t]
    assert np.all(np.abs(a1 - ref_a) <= 2.0 ** -8 * np.abs(ref_a) + 1e-30)
    assert np.all(np.abs(e1 - ref_e) <= 2.0 ** -7 * np.abs(ref_e) + 1e-30)


@pytest.mark.parametrize("D", [128, 384])
def test_filter_skips_cold_item_tiles(B, D, monkeypatch):
    # items 0..599 carry large logits, the rest near-zero ones: the softmax of every item
    # tile past the first three is far below eps, so those tiles skip their gradient work
    # while the hot tiles keep theirs. The change stays within the dropped-entry bound.
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "1024")
    eps = 2.0 ** -12
    _say(f"filter hot/cold items, D={D}")
    inp = _case(96, D, 2600, 1.0, 900 + D)
    A64, E64 = decode_inputs(inp)
    E64[600:] *= 0.03
    inp["E"] = (E64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    A64, E64 = decode_inputs(inp)
    g = upload(inp)
    a0, e0 = _grads(B, g)
    a1, e1 = _grads(B, g, eps=eps)
    b_dA, b_dE = H.ce_filter_bounds(A64, E64, inp["target"], eps)
    _check_moved(a0, a1, e0, e1, b_dA, b_dE)
    cold = np.mean(e1[768:] != e0[768:])
    print(f"[filter] cold dE rows changed: {cold:.3f}, hot: {np.mean(e1[:512] != e0[:512]):.3f}")
    assert cold > 0.5, "no cold item tile was skipped"


@pytest.mark.parametrize("D", [128, 384])
def test_filter_reused_workspace_matches_fresh(B, D, monkeypatch):
    # a hot case (large logits: many flagged tiles) and then a cold one (near-uniform softmax:
    # no dense tile reaches eps) through one workspace: the second result equals the result of
    # a fresh workspace bit for bit, so nothing of the first call's tile decisions survives
    monkeypatch.setenv("CUTLOSS_MAX_CHUNK_ITEMS", "512")
    eps = 2.0 ** -12
    _say(f"filter workspace reuse hot -> cold, D={D}")
    hot = upload(_case(96, D, 2600, 1.0, 1000 + D))
    cold = upload(_case(96, D, 2600, 0.05, 1100 + D))
    prob = B.ce_problem(hot["A"], hot["E"], hot["target"], -100)
    ws = B.workspace(max(B.cutloss_ce_workspace_size(prob, B.OP_BWD), B.cutloss_ce_workspace_size(prob, B.OP_FWD)),
                     hot["A"].device)
    ws.fill_(0x5A)                      # whatever a caller's buffer held before
    _grads(B, hot, eps=eps, ws=ws)
    a_reused, e_reused = _grads(B, cold, eps=eps, ws=ws)
    a_fresh, e_fresh = _grads(B, cold, eps=eps)
    assert np.array_equal(a_reused, a_fresh) and np.array_equal(e_reused, e_fresh)
    a_hot2, e_hot2 = _grads(B, hot, eps=eps, ws=ws)
    a_hot, e_hot = _grads(B, hot, eps=eps)
    assert np.array_equal(a_hot2, a_hot) and np.array_equal(e_hot2, e_hot)
