"""The chunked path's vocabulary plan, seen through the profiling hook's launch counts.

A backward keeps one chunk's gradient tile in the workspace. Its chunk holds at most
ceil(V / 8) items rounded up to the 256-item tile (ELMO, ai.info summary, Main Findings: the
logit buffer chunked 8 ways), so it launches the logits, dA and dE products once per chunk.
A forward stores no tile and runs the whole vocabulary as one chunk. Both sum the same
per-tile softplus partials in a fixed order, so the forward's loss and the fused backward's
loss agree to fp32 rounding (the two logits epilogues are separate instantiations, so the
compiler may contract their sums differently).
"""
from __future__ import annotations

import math

import pytest
import torch

from oracle import head_loss as H
from workloads import make
from workloads.gen import Workload

from gpu_util import canonical, check_loss, decode_inputs, dev, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def _say(msg):
    print(f"[plan] {msg}", flush=True)


@pytest.mark.parametrize("T,D,V,e_dtype", [(100, 384, 20000, "bf16"), (128, 768, 30001, "fp8"),
                                           (300, 512, 9000, "bf16")])
def test_chunk_plan_launches(B, T, D, V, e_dtype, monkeypatch):
    monkeypatch.delenv("CUTLOSS_MAX_CHUNK_ITEMS", raising=False)
    _say(f"T={T} D={D} V={V} {e_dtype}")
    w = Workload("plan", "bce", T, D, V, e_dtype, None, None, "uniform_distinct", L=6, pad_id=0,
                 mask_frac=0.1, seed=5 + D)
    inp = make(w)
    g = upload(inp)
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], 0)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD), g["A"].device)
    loss = torch.empty(T, dtype=torch.float32, device=dev())
    floss = torch.empty(T, dtype=torch.float32, device=dev())
    dA = torch.empty(T, D, dtype=torch.bfloat16, device=dev())
    dE = torch.empty(V, D, dtype=torch.bfloat16, device=dev())
    B.cutloss_profile_read()                      # drop earlier records
    B.cutloss_profile_enable(True)
    try:
        B.cutloss_bce_fwd(prob, loss, ws)
        fwd = B.cutloss_profile_read()
        B.cutloss_bce_bwd(prob, None, dA, dE, floss, ws)
        bwd = B.cutloss_profile_read()
    finally:
        B.cutloss_profile_enable(False)
    vc = math.ceil(math.ceil(V / 8) / 256) * 256
    n_chunks = math.ceil(V / vc)
    assert n_chunks >= 7
    assert fwd["chunk_logits"][1] == 1
    assert fwd["chunk_dA"][1] == 0 and fwd["chunk_dE"][1] == 0
    assert bwd["chunk_logits"][1] == n_chunks
    assert bwd["chunk_dA"][1] == n_chunks and bwd["chunk_dE"][1] == n_chunks
    assert torch.allclose(loss, floss, rtol=1e-6, atol=0.0), "forward and fused-backward losses differ"
    A64, E64 = decode_inputs(inp)
    crow, cids, _ = canonical(inp, V, 0)
    check_loss(loss.cpu().numpy(), H.bce_loss(A64, E64, crow, cids, inp["mask"]), what="loss")
    _say(f"{n_chunks} chunks of {vc} items; forward one launch")
