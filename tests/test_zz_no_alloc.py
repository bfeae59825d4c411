"""The allocation-free entry point cutloss_bce_bwd_noalloc (the library's fixed scratch
array instead of a caller workspace) against cutloss_bce_bwd with a workspace: the same
kernels on the same inputs, so the outputs agree bit for bit, and both meet the oracle's
tolerances. Two calls in a row, the second with a smaller problem, so that the second runs
on what the first left in the array; the chunked path as well (D = 384)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from workloads import make
from workloads.gen import Workload

from gpu_util import bf16_to_f64, canonical, check_grad, check_loss, decode_inputs, upload


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def test_rejects_problems_beyond_the_array_before_launch(B):
    # needs no GPU: the size check comes before any device call (fake, aligned pointers)
    p = B.BceProblem(4096, 256, 876_939, 0x10000, 0x20000, B.BF16, 0x30000, 0x40000, 32768, None, 0)
    assert B.cutloss_bce_workspace_size(p, B.OP_BWD) > B.STATIC_SCRATCH_BYTES
    lib = B.lib()
    st = lib.cutloss_bce_bwd_noalloc(ctypes.byref(p), None, ctypes.c_void_p(0x50000), ctypes.c_void_p(0x60000),
                                     ctypes.c_void_p(0x70000), None)
    assert st == B.ERR_WORKSPACE
    assert b"allocation-free" in lib.cutloss_last_error()


def _run_both(B, w, pad_id):
    inp = make(w, with_dloss=True)
    g = upload(inp)
    dev = g["A"].device
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], pad_id)
    assert B.cutloss_bce_workspace_size(prob, B.OP_BWD) <= B.STATIC_SCRATCH_BYTES
    outs = []
    for noalloc in (True, False):
        loss = torch.empty(w.T, dtype=torch.float32, device=dev)
        dA = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev)
        dE = torch.empty(w.V, w.D, dtype=torch.bfloat16, device=dev)
        if noalloc:
            B.cutloss_bce_bwd_noalloc(prob, g["dloss"], dA, dE, loss)
        else:
            ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD), dev)
            B.cutloss_bce_bwd(prob, g["dloss"], dA, dE, loss, ws)
        outs.append((loss, dA, dE))
    torch.cuda.synchronize()
    (l0, a0, e0), (l1, a1, e1) = outs
    assert torch.equal(l0, l1)
    assert torch.equal(a0.view(torch.int16), a1.view(torch.int16))
    assert torch.equal(e0.view(torch.int16), e1.view(torch.int16))
    A64, E64 = decode_inputs(inp)
    crow, cids, _ = canonical(inp, w.V, pad_id)
    check_loss(l0.cpu().numpy(), H.bce_loss(A64, E64, crow, cids, inp["mask"]), what="noalloc loss")
    dA_r, dE_r = H.bce_grads(A64, E64, crow, cids, inp["mask"], inp["dloss"])
    check_grad(bf16_to_f64(a0), dA_r, "noalloc dA")
    check_grad(bf16_to_f64(e0), dE_r, "noalloc dE")


@pytest.mark.gpu
@pytest.mark.parametrize("D,sizes", [(256, [(333, 4100), (70, 1500)]), (384, [(130, 2100), (40, 900)])])
def test_noalloc_matches_workspace_entry_point(B, D, sizes):
    for i, (T, V) in enumerate(sizes):
        print(f"[case] noalloc D={D} T={T} V={V} (call {i + 1})", flush=True)
        w = Workload("noalloc", "bce", T, D, V, "bf16", None, None, "uniform_any", L=8, pad_id=0, mask_frac=0.1,
                     seed=40 + T)
        _run_both(B, w, 0)
