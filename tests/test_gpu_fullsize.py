"""Full-size GPU parity of the remaining configurations, in the launch configuration
bench.py times, against the fp64 oracle on sampled rows and items (the oracle computes
each sample exactly; max|ref| in the gradient tolerances is the sample maximum).

* seqrec_bce_large: T = 16,384, D = 512, V = 876,939, Zipf positives, 10% masked rows
* llm_ce: T = 8,192, D = 2,304, V = 256,000 softmax CE, 5% ignored rows; dE on sampled
  items needs the logsumexp of every row, which tests/golden/make_llm_ce_lse.py computed
  once with the oracle (tests/golden/llm_ce_lse.npy)
* xmc_sgd: T = 128, D = 768, V = 3,000,000 FP8 E4M3 embeddings, fused SGD step (lr 0.01)
* cutbce_minibench: the Cut BCE mini-benchmark shape (§IV-A), T = 16,384, D = 128,
  V = 100,000 with A, E ~ N(0, I) (saturated sigmoids, large softplus terms)
Samples always include the first and last row, masked/ignored rows and rows holding
item 1; items 0, 1..8, V-1, positives and random items.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from oracle.formats import decode_bf16, decode_fp8_e4m3fn
from oracle.targets import canonical_csr
from workloads import make, workload

from gpu_util import bf16_to_f64, check_grad, check_loss, run_bce, run_ce, upload

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _rows(T, special, n_rand=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = {0, T - 1, *[int(r) for r in special]}
    rows.update(rng.choice(T, size=min(n_rand, T), replace=False).tolist())
    return np.array(sorted(rows))


def _items(V, positives, n_rand=48, seed=1):
    rng = np.random.default_rng(seed)
    items = {0, V - 1, *range(1, 9)}
    pos = np.unique(positives)
    if len(pos):
        items.update(rng.choice(pos, size=min(16, len(pos)), replace=False).tolist())
    items.update(rng.choice(V, size=n_rand, replace=False).tolist())
    return np.array(sorted(items))


def _decode_fp8_rows(E8):
    # the oracle's decoder applied to all 256 codes, then gathered (same values, less memory traffic)
    lut = decode_fp8_e4m3fn(np.arange(256, dtype=np.uint8))
    return lut[E8]


def test_seqrec_large_full_size(B):
    inp = make(workload("seqrec_bce_large"))
    w = inp["workload"]
    _say(f"seqrec_bce_large full size T={w.T} D={w.D} V={w.V}")
    out = run_bce(B, upload(inp), 0)
    A64, E64 = decode_bf16(inp["A"]), decode_bf16(inp["E"])
    crow, cids, n_bad = canonical_csr(inp["row_ptr"], inp["ids"], inp["mask"], w.V, 0)
    assert out["n_err"] == n_bad == 0
    masked = np.nonzero(inp["mask"] == 0)[0][:4]
    rp, ids = inp["row_ptr"], inp["ids"]
    with1 = [t for t in range(2000) if 1 in set(ids[rp[t]:rp[t + 1]].tolist())][:4]
    rows = _rows(w.T, list(masked) + with1)
    loss_r, dA_r = H.bce_rows(A64, E64, crow, cids, rows, inp["mask"])
    check_loss(out["loss"].cpu().numpy()[rows], loss_r, what="fwd loss (sampled rows)")
    check_loss(out["floss"].cpu().numpy()[rows], loss_r, what="fused loss (sampled rows)")
    check_grad(bf16_to_f64(out["dA"][torch.from_numpy(rows).cuda()]), dA_r, "dA (sampled rows)")
    items = _items(w.V, cids)
    dE_c = H.bce_items(A64, E64, crow, cids, items, inp["mask"])
    check_grad(bf16_to_f64(out["dE"][torch.from_numpy(items).cuda()]), dE_c, "dE (sampled items)")


def test_cutbce_minibench_full_size(B):
    inp = make(workload("cutbce_minibench"))
    w = inp["workload"]
    _say(f"cutbce_minibench full size T={w.T} D={w.D} V={w.V}")
    out = run_bce(B, upload(inp), -1)
    A64, E64 = decode_bf16(inp["A"]), decode_bf16(inp["E"])
    crow, cids, n_bad = canonical_csr(inp["row_ptr"], inp["ids"], inp["mask"], w.V, -1)
    assert out["n_err"] == n_bad == 0
    rp, ids = inp["row_ptr"], inp["ids"]
    with0 = [t for t in range(4000) if 0 in set(ids[rp[t]:rp[t + 1]].tolist())][:4]
    rows = _rows(w.T, with0)
    loss_r, dA_r = H.bce_rows(A64, E64, crow, cids, rows, inp["mask"])
    check_loss(out["loss"].cpu().numpy()[rows], loss_r, what="fwd loss (sampled rows)")
    check_loss(out["floss"].cpu().numpy()[rows], loss_r, what="fused loss (sampled rows)")
    check_grad(bf16_to_f64(out["dA"][torch.from_numpy(rows).cuda()]), dA_r, "dA (sampled rows)")
    items = _items(w.V, cids)
    dE_c = H.bce_items(A64, E64, crow, cids, items, inp["mask"])
    check_grad(bf16_to_f64(out["dE"][torch.from_numpy(items).cuda()]), dE_c, "dE (sampled items)")


def test_llm_ce_full_size(B):
    inp = make(workload("llm_ce"))
    w = inp["workload"]
    _say(f"llm_ce full size T={w.T} D={w.D} V={w.V}")
    out = run_ce(B, upload(inp))
    A64, E64 = decode_bf16(inp["A"]), decode_bf16(inp["E"])
    tgt = inp["target"]
    ignored = np.nonzero(tgt == -100)[0][:4]
    rows = _rows(w.T, ignored)
    loss_r, lse_r, dA_r = H.ce_rows(A64, E64, tgt, rows)
    check_loss(out["lse"].cpu().numpy()[rows], lse_r, what="lse (sampled rows)")
    check_loss(out["loss"].cpu().numpy()[rows], loss_r, what="loss (sampled rows)")
    check_grad(bf16_to_f64(out["dA"][torch.from_numpy(rows).cuda()]), dA_r, "dA (sampled rows)")
    lse_all = np.load(os.path.join(GOLDEN, "llm_ce_lse.npy"))
    assert lse_all.shape == (w.T,)
    np.testing.assert_allclose(lse_all[rows], lse_r, rtol=1e-12)
    items = _items(w.V, tgt[tgt >= 0])
    dE_c = H.ce_items(A64, E64, tgt, items, lse_all)
    check_grad(bf16_to_f64(out["dE"][torch.from_numpy(items).cuda()]), dE_c, "dE (sampled items)")


def test_xmc_sgd_full_size(B):
    inp = make(workload("xmc_sgd"))
    w = inp["workload"]
    _say(f"xmc_sgd full size T={w.T} D={w.D} V={w.V} fp8 E, lr={w.lr}")
    g = upload(inp)
    dev = g["A"].device
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], -1)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD_SGD), dev)
    loss_f = torch.empty(w.T, dtype=torch.float32, device=dev)
    B.cutloss_bce_fwd(prob, loss_f, ws)
    loss = torch.empty(w.T, dtype=torch.float32, device=dev)
    dA = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev)
    B.cutloss_bce_bwd_sgd(prob, None, w.lr, dA, loss, ws)
    torch.cuda.synchronize()
    assert B.cutloss_read_data_errors(ws) == 0
    A64 = decode_bf16(inp["A"])
    E64 = _decode_fp8_rows(inp["E"])
    crow, cids, _ = canonical_csr(inp["row_ptr"], inp["ids"], inp["mask"], w.V, -1)
    rows = _rows(w.T, [], n_rand=24)
    loss_r, dA_r = H.bce_rows(A64, E64, crow, cids, rows, inp["mask"])
    check_loss(loss_f.cpu().numpy()[rows], loss_r, what="fwd loss (sampled rows)")
    check_loss(loss.cpu().numpy()[rows], loss_r, what="fused SGD loss (sampled rows)")
    check_grad(bf16_to_f64(dA[torch.from_numpy(rows).cuda()]), dA_r, "dA (sampled rows)")
    items = _items(w.V, cids)
    dE_c = H.bce_items(A64, E64, crow, cids, items, inp["mask"])
    E_new = g["E"][torch.from_numpy(items).cuda()].cpu().numpy()
    from test_gpu_parity import _check_sgd
    _check_sgd(E_new, inp["E"][items], dE_c, w.lr)
