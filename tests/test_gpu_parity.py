"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Small cases run the full oracle (materialized logits) at sizes that still span
several 128-row / 32-column tiles and ragged tails; the headline workload runs at
full size and is compared on sampled rows and items, which the oracle computes
one by one. Tolerances are those of tests/gpu_util.py.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from oracle.targets import canonical_csr, item_major
from workloads import make, workload
from workloads.gen import Workload

from gpu_util import (bf16_to_f64, canonical, check_grad, check_loss, decode_inputs, run_bce, run_ce,
                       upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import binding
    return binding


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _bce_full_check(B, inp, pad_id, dloss=None, loss_only=False):
    w = inp["workload"]
    A64, E64 = decode_inputs(inp)
    crow, cids, n_bad = canonical(inp, w.V, pad_id)
    g = upload(inp)
    dl = None if dloss is None else torch.from_numpy(dloss).to(g["A"].device)
    out = run_bce(B, g, pad_id, dloss=dl, want_dA=not loss_only, want_dE=not loss_only, fused_loss=not loss_only)
    ref_loss = H.bce_loss(A64, E64, crow, cids, inp["mask"])
    check_loss(out["loss"].cpu().numpy(), ref_loss, what="fwd loss")
    assert out["n_err"] == n_bad
    if loss_only:
        return
    check_loss(out["floss"].cpu().numpy(), ref_loss, what="fused loss")
    dA, dE = H.bce_grads(A64, E64, crow, cids, inp["mask"], dloss)
    check_grad(bf16_to_f64(out["dA"]), dA, "dA")
    check_grad(bf16_to_f64(out["dE"]), dE, "dE")
    # masked rows: exact zeros
    m = inp["mask"] == 0
    if m.any():
        assert np.all(out["loss"].cpu().numpy()[m] == 0)
        assert np.all(bf16_to_f64(out["dA"])[m] == 0)


def test_tiny_bce_full(B):
    _say("tiny_bce T=32 D=64 V=1000")
    inp = make(workload("tiny_bce"), with_dloss=True)
    _bce_full_check(B, inp, pad_id=0)
    _bce_full_check(B, inp, pad_id=0, dloss=inp["dloss"])


# T = 333 at D = 256 gives two 256-row workgroups of the rows sweep, the second one ragged
# in both its leading and its lagging half of waves
@pytest.mark.parametrize("T,D,V", [(1, 64, 33), (33, 128, 1001), (130, 256, 4097), (333, 256, 2531), (257, 64, 2000),
                                   (129, 512, 777)])
def test_bce_ragged_with_pads_and_repeats(B, T, D, V):
    _say(f"ragged T={T} D={D} V={V}")
    w = Workload("ragged", "bce", T, D, V, "bf16", None, None, "uniform_any", L=12, pad_id=0, mask_frac=0.2,
                 seed=100 + T)
    inp = make(w, with_dloss=True)
    _bce_full_check(B, inp, pad_id=0, dloss=inp["dloss"])


@pytest.mark.parametrize("T,D", [(96, 128), (300, 256)])
def test_bce_high_scale_stress(B, T, D):
    # Cut BCE §IV-A mini-benchmark distribution: A, E ~ N(0, I), L = 8 uniform targets in
    # [0, V) (pads and repeats included): saturated sigmoids, large softplus.
    _say(f"stress N(0,1) T={T} D={D} V=5000")
    w = Workload("stress", "bce", T, D, 5000, "bf16", 1.0, 1.0, "uniform_any", L=8, pad_id=0, seed=7 + D)
    inp = make(w)
    _bce_full_check(B, inp, pad_id=0)


@pytest.mark.parametrize("T,D", [(70, 128), (270, 256)])
def test_bce_closed_forms(B, T, D):
    # A = 0: loss = V ln 2, dA_t = 0.5 sum_v E_v - sum_p E_p, dE = 0
    # E = 0: loss = V ln 2, dA = 0, dE_v = sum_t w_t (0.5 - y_tv) A_t
    w = Workload("cf", "bce", T, D, 3000, "bf16", None, None, "uniform_any", L=6, pad_id=0, mask_frac=0.1,
                 seed=8 if D == 128 else 9)
    inp = make(w)
    for zero in ("A", "E"):
        _say(f"closed form {zero}=0")
        z = dict(inp)
        z[zero] = np.zeros_like(inp[zero])
        _bce_full_check(B, z, pad_id=0)
        out = run_bce(B, upload(z), 0)
        valid = z["mask"] != 0
        np.testing.assert_allclose(out["loss"].cpu().numpy()[valid], w.V * math.log(2.0), rtol=1e-5)


# up to 4,096 IDs and 8,192 rows: one workgroup sorts them in LDS; 6,000 IDs: the radix
# passes form their own block offsets; 150,000 IDs (147 sort blocks of 1,024): the
# histograms are scanned by a kernel of their own
@pytest.mark.parametrize("T,V,L", [(1, 50, 40), (200, 3000, 15), (300, 5000, 20), (3000, 200_000, 50)])
def test_canonical_targets_bit_exact(B, T, V, L):
    _say(f"canonical targets T={T} V={V} L={L}")
    w = Workload("canon", "bce", T, 64, V, "bf16", None, None, "uniform_any", L=L, pad_id=0, mask_frac=0.3, seed=9)
    inp = make(w)
    # plant out-of-range IDs and an empty row
    ids = inp["ids"].copy()
    ids[::37] = V + np.arange(len(ids[::37]))
    ids[5::41] = -3
    inp["ids"] = ids
    g = upload(inp)
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], 0)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD), g["A"].device)
    n = len(ids)
    dev = g["A"].device
    crow = torch.empty(w.T + 1, dtype=torch.int32, device=dev)
    cids, items, rows = (torch.empty(n, dtype=torch.int32, device=dev) for _ in range(3))
    nu = B.cutloss_bce_canonical_targets(prob, crow, cids, items, rows, ws)
    ref_crow, ref_cids, n_bad = canonical_csr(inp["row_ptr"], ids, inp["mask"], w.V, 0)
    ref_items, ref_rows = item_major(ref_crow, ref_cids)
    assert nu == len(ref_cids)
    assert np.array_equal(crow.cpu().numpy(), ref_crow)
    assert np.array_equal(cids.cpu().numpy()[:nu], ref_cids)
    assert np.array_equal(items.cpu().numpy()[:nu], ref_items)
    assert np.array_equal(rows.cpu().numpy()[:nu], ref_rows)
    assert B.cutloss_read_data_errors(ws) == n_bad and n_bad > 0


def _targets_model(row_ptr, ids, mask, V, pad, nnz):
    """The canonicalization's documented handling of malformed input, row by row: a row with
    b < 0, e > nnz or e < b is one data error and has no positives; IDs outside [0, V) are
    errors; valid entries are laid out in row order and cut at nnz (overlapping rows of a
    non-monotone row_ptr), the excess counted as errors; repeats count once."""
    T = len(row_ptr) - 1
    cnt, bad = [], 0
    for t in range(T):
        b, e = int(row_ptr[t]), int(row_ptr[t + 1])
        if b < 0 or e > nnz or e < b:
            bad += 1
            cnt.append(0)
            continue
        c = 0
        if mask[t]:
            for i in range(b, e):
                v = int(ids[i])
                if pad >= 0 and v == pad:
                    continue
                if v < 0 or v >= V:
                    bad += 1
                    continue
                c += 1
        cnt.append(c)
    off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)
    pairs = [None] * nnz
    for t in range(T):
        if cnt[t] == 0:
            continue
        o = int(off[t])
        for i in range(int(row_ptr[t]), int(row_ptr[t + 1])):
            v = int(ids[i])
            if (pad >= 0 and v == pad) or v < 0 or v >= V:
                continue
            if o >= nnz:
                break
            pairs[o] = (v, t)
            o += 1
    total = int(off[-1])
    n0 = min(total, nnz)
    bad += total - n0
    uniq = sorted(set(pairs[:n0]))                        # (item, row)
    by_row = sorted((r, v) for v, r in uniq)
    crow = np.zeros(T + 1, dtype=np.int64)
    for r, _ in by_row:
        crow[r + 1] += 1
    crow = np.cumsum(crow)
    cids = np.array([v for _, v in by_row], dtype=np.int64)
    items = np.array([v for v, _ in uniq], dtype=np.int64)
    rows = np.array([r for _, r in uniq], dtype=np.int64)
    return crow, cids, items, rows, bad


# malformed rows (e < b, e > nnz) and overlapping rows whose entries exceed nnz: the
# single-workgroup path (500 IDs) and the radix pipeline (6,000 IDs) give the model's result
@pytest.mark.parametrize("T,L", [(50, 10), (600, 10)])
def test_canonical_targets_malformed_rows(B, T, L):
    _say(f"canonical targets, malformed rows T={T} L={L}")
    rng = np.random.default_rng(31 + T)
    V = 4000
    lens = rng.integers(0, 2 * L, size=T)
    lens[0] = 2 * L
    lens[-1] = 0
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    nnz = int(row_ptr[-1])
    ids = rng.integers(-2, V + 3, size=nnz).astype(np.int32)
    k = T // 5
    row_ptr[k] = row_ptr[k + 1] + 20                      # row k - 1 overlaps, row k has e < b
    row_ptr[T] = nnz + 5                                  # the last row ends past nnz
    mask = np.ones(T, dtype=np.uint8)                     # every row counts, so the overlap exceeds nnz
    dev = torch.device("cuda:0")
    A = torch.zeros(T, 64, dtype=torch.bfloat16, device=dev)
    E = torch.zeros(V, 64, dtype=torch.bfloat16, device=dev)
    g_rp = torch.from_numpy(row_ptr).to(dev)
    g_ids = torch.from_numpy(ids).to(dev)
    g_mask = torch.from_numpy(mask).to(dev)
    prob = B.bce_problem(A, E, g_rp, g_ids, g_mask, 0)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD), dev)
    crow = torch.empty(T + 1, dtype=torch.int32, device=dev)
    cids, items, rows = (torch.empty(nnz, dtype=torch.int32, device=dev) for _ in range(3))
    nu = B.cutloss_bce_canonical_targets(prob, crow, cids, items, rows, ws)
    ref_crow, ref_cids, ref_items, ref_rows, ref_bad = _targets_model(row_ptr, ids, mask, V, 0, nnz)
    assert ref_bad >= 10                                  # two malformed rows and the entries cut at nnz
    assert nu == len(ref_cids)
    assert np.array_equal(crow.cpu().numpy(), ref_crow)
    assert np.array_equal(cids.cpu().numpy()[:nu], ref_cids)
    assert np.array_equal(items.cpu().numpy()[:nu], ref_items)
    assert np.array_equal(rows.cpu().numpy()[:nu], ref_rows)
    assert B.cutloss_read_data_errors(ws) == ref_bad


def test_determinism(B):
    _say("determinism")
    w = Workload("det", "bce", 200, 256, 9000, "bf16", None, None, "zipf", L=8, pad_id=0, mask_frac=0.1, seed=11)
    g = upload(make(w))
    a = run_bce(B, g, 0)
    b = run_bce(B, g, 0)
    for k in ("loss", "dA", "dE", "floss"):
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k]), k


@pytest.mark.parametrize("T,D,V", [(70, 128, 3001), (200, 256, 5000), (300, 256, 2049), (33, 64, 100)])
def test_ce_small(B, T, D, V):
    _say(f"ce T={T} D={D} V={V}")
    w = Workload("ce", "ce", T, D, V, "bf16", None, None, "ce_uniform", L=1, pad_id=-1, ignore_frac=0.1, seed=12 + T)
    inp = make(w, with_dloss=True)
    tgt = inp["target"].copy()
    tgt[3] = V + 5          # out of range: counted, row ignored
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


@pytest.mark.parametrize("D", [128, 256])
def test_sgd_fp8_small(B, D):
    _say(f"sgd fp8 T=40 D={D} V=2000")
    w = Workload("sgd", "bce", 40, D, 2000, "fp8", None, 0.05, "poisson_distinct", L=5, pad_id=-1, lr=0.01,
                 seed=13 if D == 128 else 14)
    inp = make(w)
    A64, E64 = decode_inputs(inp)
    crow, cids, _ = canonical(inp, w.V, -1)
    g = upload(inp)
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], -1)
    # one workspace for the unfused backward and the SGD step: large enough for both
    ws = B.workspace(max(B.cutloss_bce_workspace_size(prob, B.OP_BWD), B.cutloss_bce_workspace_size(prob, B.OP_BWD_SGD)),
                     g["A"].device)
    # unfused dE on the same fp8 E first
    dE = torch.empty(w.V, w.D, dtype=torch.bfloat16, device=g["A"].device)
    B.cutloss_bce_bwd(prob, None, None, dE, None, ws)
    loss = torch.empty(w.T, dtype=torch.float32, device=g["A"].device)
    B.cutloss_bce_bwd_sgd(prob, None, w.lr, None, loss, ws)
    torch.cuda.synchronize()
    _, dE_ref = H.bce_grads(A64, E64, crow, cids, inp["mask"])
    check_grad(bf16_to_f64(dE), dE_ref, "dE (fp8 E)")
    check_loss(loss.cpu().numpy(), H.bce_loss(A64, E64, crow, cids, inp["mask"]), what="sgd fused loss")
    _check_sgd(g["E"].cpu().numpy(), inp["E"], dE_ref, w.lr)


def _check_sgd(E_new, E_old, dE_ref, lr, fmt="fp8", max_frac=1e-2):
    """E' must be round(E - lr (dE_ref + delta)) for some |delta| <= 2e-2 max|dE_ref| per
    element (round: nearest-even onto E's grid, FP8 E4M3FN or bf16); fewer than max_frac of
    the elements may differ from round(E - lr dE_ref) itself."""
    from oracle.formats import decode_bf16, decode_fp8_e4m3fn
    sgd, dec = (H.sgd_fp8, decode_fp8_e4m3fn) if fmt == "fp8" else (H.sgd_bf16, decode_bf16)
    tol = 2e-2 * np.abs(dE_ref).max()
    lo = sgd(E_old, dE_ref + tol, lr)
    hi = sgd(E_old, dE_ref - tol, lr)
    got = dec(E_new)
    vlo, vhi = dec(lo), dec(hi)
    assert np.all((got >= vlo) & (got <= vhi)), "SGD result outside the rounding interval"
    exact = dec(sgd(E_old, dE_ref, lr))
    frac = float(np.mean(got != exact))
    print(f"[sgd] fraction differing from {fmt}(E - lr dE_ref): {frac:.2e}")
    assert frac < max_frac


@pytest.mark.parametrize("D", [64, 128, 256])
def test_sgd_bf16_fused_sweeps(B, D):
    """bf16 E at D in {64, 128, 256}: the cols sweep applies E <- bf16(E - lr dE) in place
    in its epilogue (dE never stored); the rows sweep of the same call reads E first."""
    _say(f"sgd bf16 T=150 D={D} V=3000 (fused sweeps)")
    w = Workload("sgd_bf16", "bce", 150, D, 3000, "bf16", None, None, "poisson_distinct", L=5, pad_id=-1, lr=0.01,
                 mask_frac=0.1, seed=15 if D == 128 else 16)
    inp = make(w)
    A64, E64 = decode_inputs(inp)
    crow, cids, _ = canonical(inp, w.V, -1)
    g = upload(inp)
    dev = g["A"].device
    prob = B.bce_problem(g["A"], g["E"], g["row_ptr"], g["ids"], g["mask"], -1)
    # one workspace for the unfused backward and the SGD step: large enough for both
    ws = B.workspace(max(B.cutloss_bce_workspace_size(prob, B.OP_BWD), B.cutloss_bce_workspace_size(prob, B.OP_BWD_SGD)),
                     dev)
    dE = torch.empty(w.V, w.D, dtype=torch.bfloat16, device=dev)
    B.cutloss_bce_bwd(prob, None, None, dE, None, ws)
    loss = torch.empty(w.T, dtype=torch.float32, device=dev)
    dA = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev)
    B.cutloss_bce_bwd_sgd(prob, None, w.lr, dA, loss, ws)
    torch.cuda.synchronize()
    dA_ref, dE_ref = H.bce_grads(A64, E64, crow, cids, inp["mask"])
    check_grad(bf16_to_f64(dE), dE_ref, "dE (bf16 E, unfused)")
    check_grad(bf16_to_f64(dA), dA_ref, "dA (fused SGD call, old E)")
    check_loss(loss.cpu().numpy(), H.bce_loss(A64, E64, crow, cids, inp["mask"]), what="sgd fused loss")
    E_new = g["E"].view(torch.int16).cpu().numpy().view(np.uint16)
    # bf16's grid is 32x finer than E4M3's: a larger share of the steps sits near a rounding
    # boundary within the gradient tolerance
    _check_sgd(E_new, inp["E"], dE_ref, w.lr, fmt="bf16", max_frac=0.15)
    # masked rows and rows with no positive still move E through the dense term only
    assert not np.array_equal(E_new, inp["E"])


# ----------------------------------------------------------------------------- full size

def _sample_rows(inp, T, n_rand=64, seed=0):
    rng = np.random.default_rng(seed)
    rows = {0, T - 1}
    masked = np.nonzero(inp["mask"] == 0)[0]
    rows.update(masked[:4].tolist())
    rp, ids = inp["row_ptr"], inp["ids"]
    with1 = [t for t in range(min(T, 2000)) if 1 in set(ids[rp[t]:rp[t + 1]].tolist())]
    rows.update(with1[:4])
    rows.update(rng.choice(T, size=min(n_rand, T), replace=False).tolist())
    return np.array(sorted(rows))


def _sample_items(cids, V, n_rand=64, seed=1):
    rng = np.random.default_rng(seed)
    items = {0, V - 1, *range(1, 9)}
    pos = np.unique(cids)
    items.update(rng.choice(pos, size=min(16, len(pos)), replace=False).tolist())
    items.update(rng.choice(V, size=n_rand, replace=False).tolist())
    return np.array(sorted(items))


@pytest.fixture(scope="module")
def seqrec():
    return make(workload("seqrec_bce"))


def test_seqrec_full_size_fused_fwd_bwd(B, seqrec):
    """T=4096, D=256, V=876,939, Zipf positives, 10% masked rows: the headline workload,
    run in the same launch configuration the benchmark times (fused backward with loss)."""
    inp = seqrec
    w = inp["workload"]
    _say(f"seqrec full size T={w.T} D={w.D} V={w.V}")
    g = upload(inp)
    out = run_bce(B, g, 0)
    A64, E64 = decode_inputs(inp)
    crow, cids, n_bad = canonical(inp, w.V, 0)
    assert out["n_err"] == n_bad == 0
    rows = _sample_rows(inp, w.T)
    items = _sample_items(cids, w.V)
    loss_r, dA_r = H.bce_rows(A64, E64, crow, cids, rows, inp["mask"])
    check_loss(out["loss"].cpu().numpy()[rows], loss_r, what="fwd loss (sampled rows)")
    check_loss(out["floss"].cpu().numpy()[rows], loss_r, what="fused loss (sampled rows)")
    check_grad(bf16_to_f64(out["dA"][torch.from_numpy(rows).cuda()]), dA_r, "dA (sampled rows)")
    dE_c = H.bce_items(A64, E64, crow, cids, items, inp["mask"])
    check_grad(bf16_to_f64(out["dE"][torch.from_numpy(items).cuda()]), dE_c, "dE (sampled items)")
    # the positive terms on their own scale: item sums of the sparse dE term show in items 1..8
    m = inp["mask"] == 0
    assert np.all(out["loss"].cpu().numpy()[m] == 0) and np.all(out["floss"].cpu().numpy()[m] == 0)
