"""Pins of the oracle's BCE / CE / SGD definitions.

Each pin is independent of the oracle's own formula: closed forms at A = 0 and
E = 0 (worked out by hand, evaluated with explicit loops), torch's library
BCE-with-logits / cross-entropy with autograd, central finite differences,
the dense+sparse identity named by Cut BCE §I-B, invariants, and the printed
logit-memory figure of Cut BCE §I-A.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import head_loss as H
from oracle.formats import decode_fp8_e4m3fn, encode_fp8_e4m3fn
from oracle.targets import canonical_csr, dense_labels


def _problem(T, D, V, seed, std=None, L=4, pad=0, mask_frac=0.25):
    rng = np.random.default_rng(seed)
    s = 1.0 / math.sqrt(D) if std is None else std
    A = rng.normal(0, s, (T, D))
    E = rng.normal(0, s, (V, D))
    rows = [rng.integers(0, V, size=L).tolist() for _ in range(T)]   # pads, repeats allowed
    row_ptr = np.zeros(T + 1, np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    ids = np.array([v for r in rows for v in r], np.int64)
    mask = (rng.random(T) >= mask_frac).astype(np.uint8)
    crow, cids, _ = canonical_csr(row_ptr, ids, mask, V, pad)
    w = rng.uniform(0.5, 1.5, T)
    return A, E, crow, cids, mask, w


# ---------------------------------------------------------------------------- BCE

def test_bce_closed_form_at_A_zero():
    T, D, V = 6, 5, 23
    _, E, crow, cids, mask, w = _problem(T, D, V, 0)
    A = np.zeros((T, D))
    loss = H.bce_loss(A, E, crow, cids, mask)
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w)
    for t in range(T):
        want_loss = V * math.log(2.0) if mask[t] else 0.0
        assert loss[t] == pytest.approx(want_loss, rel=1e-14, abs=0)
        want = np.zeros(D)
        if mask[t]:
            for v in range(V):
                want += 0.5 * E[v]
            for p in cids[crow[t]:crow[t + 1]]:
                want -= E[p]
            want *= w[t]
        np.testing.assert_allclose(dA[t], want, rtol=1e-12, atol=1e-13)
    assert np.all(dE == 0)


def test_bce_closed_form_at_E_zero():
    T, D, V = 7, 4, 19
    A, _, crow, cids, mask, w = _problem(T, D, V, 1)
    E = np.zeros((V, D))
    loss = H.bce_loss(A, E, crow, cids, mask)
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w)
    np.testing.assert_allclose(loss, np.where(mask != 0, V * math.log(2.0), 0.0), rtol=1e-14)
    assert np.all(dA == 0)
    for v in range(V):
        want = np.zeros(D)
        for t in range(T):
            if not mask[t]:
                continue
            y = 1.0 if v in set(cids[crow[t]:crow[t + 1]].tolist()) else 0.0
            want += w[t] * (0.5 - y) * A[t]
        np.testing.assert_allclose(dE[v], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("std", [None, 1.0, 4.0])
def test_bce_dense_sparse_identity(std):
    # Cut BCE §I-B: exact split into dense background and sparse correction;
    # std=1.0, D=128 is the mini-benchmark's A, E ~ N(0, I) (§IV-A)
    T, D, V = 9, 128, 301
    A, E, crow, cids, mask, _ = _problem(T, D, V, 2, std=std, L=8)
    a = H.bce_loss(A, E, crow, cids, mask)
    b = H.bce_loss_dense_sparse(A, E, crow, cids, mask)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def _torch_bce(A, E, crow, cids, mask, w):
    T, V = A.shape[0], E.shape[0]
    At = torch.tensor(A, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    X = At @ Et.T
    Y = torch.tensor(dense_labels(crow, cids, T, V))
    per = torch.nn.functional.binary_cross_entropy_with_logits(X, Y, reduction="none").sum(1)
    per = per * torch.tensor(mask, dtype=torch.float64)
    (per * torch.tensor(w)).sum().backward()
    return per.detach().numpy(), At.grad.numpy(), Et.grad.numpy()


def test_positive_logits_by_brute_force_and_torch_bce():
    # Cut BCE §I-B: the sparse correction's terms x_tp = A_t . E_p, pinned two ways: a
    # scalar loop over (t, p, d) on the canonical pairs, and the split of torch's library
    # BCE loss, sum_v softplus(x_tv) - loss_t = sum_p x_tp for every valid row
    T, D, V = 7, 5, 29
    A, E, crow, cids, mask, w = _problem(T, D, V, 11, std=0.9, L=6)
    x_pos, sum_x = H.positive_logits(A, E, crow, cids)
    assert x_pos.shape == (len(cids),) and sum_x.shape == (T,)
    for t in range(T):
        acc_row = 0.0
        for e in range(crow[t], crow[t + 1]):
            acc = 0.0
            for d in range(D):
                acc += A[t, d] * E[cids[e], d]
            assert x_pos[e] == pytest.approx(acc, rel=1e-13, abs=1e-15)
            acc_row += acc
        assert sum_x[t] == pytest.approx(acc_row, rel=1e-13, abs=1e-15)
    assert np.all(sum_x[mask == 0] == 0)      # masked rows keep no canonical positives
    loss_t, _, _ = _torch_bce(A, E, crow, cids, np.ones(T, np.uint8), np.ones(T))
    dense = torch.nn.functional.softplus(torch.tensor(A @ E.T)).sum(1).numpy()
    np.testing.assert_allclose(dense - loss_t, sum_x, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed,std", [(3, None), (4, 1.0), (5, 3.0)])
def test_bce_matches_torch_library_and_autograd(seed, std):
    T, D, V = 8, 16, 77
    A, E, crow, cids, mask, w = _problem(T, D, V, seed, std=std)
    loss_t, dA_t, dE_t = _torch_bce(A, E, crow, cids, mask, w)
    loss = H.bce_loss(A, E, crow, cids, mask)
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w)
    np.testing.assert_allclose(loss, loss_t, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, dA_t, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dE, dE_t, rtol=1e-10, atol=1e-12)


def test_bce_finite_differences():
    T, D, V = 3, 6, 37
    A, E, crow, cids, mask, w = _problem(T, D, V, 6, std=0.7, mask_frac=0.0)
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w)
    L = lambda A_, E_: float((w * H.bce_loss(A_, E_, crow, cids, mask)).sum())
    h = 1e-6
    for (t, d) in [(0, 0), (1, 3), (2, 5)]:
        Ap, Am = A.copy(), A.copy()
        Ap[t, d] += h
        Am[t, d] -= h
        assert (L(Ap, E) - L(Am, E)) / (2 * h) == pytest.approx(dA[t, d], rel=1e-6, abs=1e-8)
    for (v, d) in [(0, 1), (int(cids[0]), 2), (36, 5)]:
        Ep, Em = E.copy(), E.copy()
        Ep[v, d] += h
        Em[v, d] -= h
        assert (L(A, Ep) - L(A, Em)) / (2 * h) == pytest.approx(dE[v, d], rel=1e-6, abs=1e-8)


def test_bce_invariants():
    T, D, V = 10, 8, 40
    rng = np.random.default_rng(7)
    A, E, crow, cids, mask, w = _problem(T, D, V, 7, std=0.5, L=5)
    loss = H.bce_loss(A, E, crow, cids, mask)
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w)
    # masked rows: exact zeros
    assert np.all(loss[mask == 0] == 0) and np.all(dA[mask == 0] == 0)
    # permuting E rows together with relabelled ids
    perm = rng.permutation(V)
    inv = np.argsort(perm)                  # new id of old item v is inv[v]
    E2 = E[perm]
    cids2 = inv[cids]
    crow2 = crow
    # re-sort each row to keep the canonical order
    cids2 = np.concatenate([np.sort(cids2[crow[t]:crow[t + 1]]) for t in range(T)])
    np.testing.assert_allclose(H.bce_loss(A, E2, crow2, cids2, mask), loss, rtol=1e-12)
    dA2, dE2 = H.bce_grads(A, E2, crow2, cids2, mask, w)
    np.testing.assert_allclose(dA2, dA, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dE2, dE[perm], rtol=1e-10, atol=1e-13)
    # permuting rows permutes outputs
    rp = rng.permutation(T)
    sets = [cids[crow[t]:crow[t + 1]] for t in range(T)]
    crow3 = np.zeros(T + 1, np.int64)
    crow3[1:] = np.cumsum([len(sets[t]) for t in rp])
    cids3 = np.concatenate([sets[t] for t in rp])
    np.testing.assert_allclose(H.bce_loss(A[rp], E, crow3, cids3, mask[rp]), loss[rp], rtol=1e-12)
    # a positive changes the loss by exactly -x (dense part unchanged)
    X = A @ E.T
    t = int(np.nonzero(mask)[0][0])
    extra = [v for v in range(V) if v not in set(sets[t].tolist())][0]
    sets4 = list(sets)
    sets4[t] = np.sort(np.append(sets[t], extra))
    crow4 = np.zeros(T + 1, np.int64)
    crow4[1:] = np.cumsum([len(s) for s in sets4])
    loss4 = H.bce_loss(A, E, crow4, np.concatenate(sets4), mask)
    assert loss4[t] - loss[t] == pytest.approx(-X[t, extra], rel=1e-9, abs=1e-12)


def test_bce_sampled_equals_full():
    T, D, V = 12, 8, 50
    A, E, crow, cids, mask, w = _problem(T, D, V, 8)
    loss = H.bce_loss(A, E, crow, cids, mask)
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w)
    rows = np.array([0, 5, 11, 3])
    items = np.array([0, 1, 49, 17, int(cids[0])])
    lr, dAr = H.bce_rows(A, E, crow, cids, rows, mask, w)
    dEc = H.bce_items(A, E, crow, cids, items, mask, w)
    np.testing.assert_allclose(lr, loss[rows], rtol=1e-13)
    np.testing.assert_allclose(dAr, dA[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dEc, dE[items], rtol=1e-12, atol=1e-15)


def test_logit_memory_formula_matches_printed_figure():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "logit_memory.json")))
    gib = H.logits_bytes_fp32(g["B_local"] * g["N"], g["V"]) / 2 ** 30
    assert round(gib, 2) == g["gib_printed"]


# ---------------------------------------------------------------------------- CE

def _ce_problem(T, D, V, seed, std=None, ign=2):
    rng = np.random.default_rng(seed)
    s = 1.0 / math.sqrt(D) if std is None else std
    A = rng.normal(0, s, (T, D))
    E = rng.normal(0, s, (V, D))
    tgt = rng.integers(0, V, T)
    tgt[rng.permutation(T)[:ign]] = -100
    return A, E, tgt, rng.uniform(0.5, 1.5, T)


def test_ce_closed_form_at_A_zero():
    T, D, V = 5, 4, 31
    _, E, tgt, w = _ce_problem(T, D, V, 10)
    A = np.zeros((T, D))
    loss, lse = H.ce_forward(A, E, tgt)
    np.testing.assert_allclose(lse, math.log(V), rtol=1e-14)
    dA, dE = H.ce_grads(A, E, tgt, dloss=w)
    for t in range(T):
        if tgt[t] == -100:
            assert loss[t] == 0 and np.all(dA[t] == 0)
            continue
        assert loss[t] == pytest.approx(math.log(V), rel=1e-14)
        want = w[t] * (sum(E[v] for v in range(V)) / V - E[tgt[t]])
        np.testing.assert_allclose(dA[t], want, rtol=1e-12, atol=1e-14)
    assert np.all(dE == 0)


@pytest.mark.parametrize("seed,std", [(11, None), (12, 1.0)])
def test_ce_matches_torch_library_and_autograd(seed, std):
    T, D, V = 9, 16, 67
    A, E, tgt, w = _ce_problem(T, D, V, seed, std=std)
    At = torch.tensor(A, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    per = torch.nn.functional.cross_entropy(At @ Et.T, torch.tensor(tgt), ignore_index=-100, reduction="none")
    (per * torch.tensor(w)).sum().backward()
    loss, lse = H.ce_forward(A, E, tgt)
    dA, dE = H.ce_grads(A, E, tgt, dloss=w)
    np.testing.assert_allclose(loss, per.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.tensor(A @ E.T), 1).numpy(), rtol=1e-13)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dE, Et.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_ce_finite_differences():
    T, D, V = 3, 5, 29
    A, E, tgt, w = _ce_problem(T, D, V, 13, std=0.8, ign=1)
    dA, dE = H.ce_grads(A, E, tgt, dloss=w)
    L = lambda A_, E_: float((w * H.ce_forward(A_, E_, tgt)[0]).sum())
    h = 1e-6
    for (t, d) in [(0, 0), (1, 2), (2, 4)]:
        Ap, Am = A.copy(), A.copy()
        Ap[t, d] += h
        Am[t, d] -= h
        assert (L(Ap, E) - L(Am, E)) / (2 * h) == pytest.approx(dA[t, d], rel=1e-6, abs=1e-9)
    for (v, d) in [(0, 0), (int(tgt[tgt >= 0][0]), 3), (28, 1)]:
        Ep, Em = E.copy(), E.copy()
        Ep[v, d] += h
        Em[v, d] -= h
        assert (L(A, Ep) - L(A, Em)) / (2 * h) == pytest.approx(dE[v, d], rel=1e-6, abs=1e-9)


def test_ce_sampled_equals_full():
    T, D, V = 10, 8, 45
    A, E, tgt, w = _ce_problem(T, D, V, 14)
    loss, lse = H.ce_forward(A, E, tgt)
    dA, dE = H.ce_grads(A, E, tgt, dloss=w)
    rows = np.array([0, 9, 4])
    items = np.array([0, 44, int(tgt[tgt >= 0][0])])
    lr, lser, dAr = H.ce_rows(A, E, tgt, rows, dloss=w)
    np.testing.assert_allclose(lr, loss[rows], rtol=1e-13)
    np.testing.assert_allclose(lser, lse[rows], rtol=1e-13)
    np.testing.assert_allclose(dAr, dA[rows], rtol=1e-12, atol=1e-15)
    lse_all = H.ce_lse(A, E, np.arange(T))
    np.testing.assert_allclose(H.ce_items(A, E, tgt, items, lse_all, dloss=w), dE[items], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------- SGD

def test_sgd_fp8_matches_torch_rounding():
    rng = np.random.default_rng(15)
    # lr a power of two and dE on a 2^-10 grid: E - lr dE is exact in float32, so torch's
    # float64 -> float32 -> fp8 cast rounds once, like the oracle
    E_codes = encode_fp8_e4m3fn(rng.normal(0, 0.05, (64, 32)))
    dE = np.round(rng.normal(0, 3.0, (64, 32)) * 1024) / 1024
    lr = 2.0 ** -7
    ours = H.sgd_fp8(E_codes, dE, lr)
    pre = decode_fp8_e4m3fn(E_codes) - lr * dE
    ref = torch.from_numpy(pre).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_sgd_bf16_matches_torch_rounding():
    from oracle.formats import decode_bf16
    rng = np.random.default_rng(16)
    # E on the bf16 grid near N(0, 1/16), lr a power of two, dE on a 2^-12 grid: E - lr dE is
    # exact in float32, so torch's float32 -> bfloat16 cast rounds once, like the oracle
    E32 = torch.from_numpy(rng.normal(0, 0.0625, (64, 48)).astype(np.float32)).to(torch.bfloat16)
    E_bits = E32.view(torch.int16).numpy().view(np.uint16)
    dE = np.round(rng.normal(0, 2.0, (64, 48)) * 4096) / 4096
    lr = 2.0 ** -7
    ours = H.sgd_bf16(E_bits, dE, lr)
    pre = decode_bf16(E_bits) - lr * dE
    assert np.array_equal(pre.astype(np.float32).astype(np.float64), pre)
    ref = torch.from_numpy(pre.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # lr = 0 keeps every pattern; a step of one ulp moves to the neighbouring pattern
    assert np.array_equal(H.sgd_bf16(E_bits, dE, 0.0), E_bits | 0)
    one = np.array([0x3F80], dtype=np.uint16)                  # 1.0, next pattern up is 1 + 2^-7
    assert H.sgd_bf16(one, np.array([-(2.0 ** -7)]), 1.0).tolist() == [0x3F81]


def test_ce_filter_bound_limits():
    # eps above every probability: the bound covers dropping the whole dense part, i.e. the
    # gap between the full gradient and the target-only gradient; eps = 0 bounds nothing
    rng = np.random.default_rng(11)
    T, D, V = 6, 5, 40
    A = rng.standard_normal((T, D))
    E = rng.standard_normal((V, D))
    target = rng.integers(0, V, size=T)
    target[2] = -100
    b_dA, b_dE = H.ce_filter_bounds(A, E, target, 2.0)
    dA, dE = H.ce_grads(A, E, target)
    valid = target != -100
    only_dA = np.zeros_like(dA)
    only_dE = np.zeros_like(dE)
    for t in np.nonzero(valid)[0]:
        only_dA[t] = -E[target[t]]
        only_dE[target[t]] -= A[t]
    assert np.all(np.abs(dA - only_dA) <= b_dA + 1e-12)
    assert np.all(np.abs(dE - only_dE) <= b_dE + 1e-12)
    # the bound is the triangle inequality of that gap: equal where all terms share a sign
    P = np.exp(A @ E.T - H.logsumexp_rows(A @ E.T)[:, None]) * valid[:, None]
    assert np.allclose(b_dA, P @ np.abs(E)) and np.allclose(b_dE, P.T @ np.abs(A))
    z_dA, z_dE = H.ce_filter_bounds(A, E, target, 0.0)
    assert not z_dA.any() and not z_dE.any()
    m_dA, _ = H.ce_filter_bounds(A, E, target, 0.05)
    assert np.all(m_dA <= b_dA + 1e-15)


def test_ce_filter_bound_brackets_brute_force_drop():
    # drop, by brute force on the materialized softmax, every dense entry below eps and
    # recompute both gradients: each moves by no more than the bound
    rng = np.random.default_rng(12)
    T, D, V = 7, 6, 50
    A = 1.5 * rng.standard_normal((T, D))
    E = rng.standard_normal((V, D))
    target = rng.integers(0, V, size=T)
    target[4] = -100
    eps = 0.02
    valid = target != -100
    X = A @ E.T
    S = np.exp(X - H.logsumexp_rows(X)[:, None]) * valid[:, None]
    Y = np.zeros_like(S)
    for t in np.nonzero(valid)[0]:
        Y[t, target[t]] = 1.0
    kept = np.where(S >= eps, S, 0.0)
    assert 0 < np.count_nonzero(S < eps) < S.size        # some entries dropped, some kept
    dA_full, dE_full = (S - Y) @ E, (S - Y).T @ A
    dA_drop, dE_drop = (kept - Y) @ E, (kept - Y).T @ A
    b_dA, b_dE = H.ce_filter_bounds(A, E, target, eps)
    assert np.all(np.abs(dA_full - dA_drop) <= b_dA + 1e-12)
    assert np.all(np.abs(dE_full - dE_drop) <= b_dE + 1e-12)
    assert np.allclose(dA_full, H.ce_grads(A, E, target)[0])


# ------------------------------------------------------------------ FP8 logits (ELMO)

def test_fp8_logits_reduce_to_plain_on_the_fp8_grid():
    # activations already on the E4M3FN grid: the cast changes nothing
    T, D, V = 6, 8, 31
    A, E, crow, cids, mask, w = _problem(T, D, V, 21, std=0.5)
    A8 = decode_fp8_e4m3fn(encode_fp8_e4m3fn(A))
    assert np.array_equal(H.fp8_activations(A8), A8)
    np.testing.assert_array_equal(H.bce_loss(A8, E, crow, cids, mask, A_logits=H.fp8_activations(A8)),
                                  H.bce_loss(A8, E, crow, cids, mask))
    g1 = H.bce_grads(A8, E, crow, cids, mask, w, A_logits=H.fp8_activations(A8))
    g0 = H.bce_grads(A8, E, crow, cids, mask, w)
    assert all(np.array_equal(a, b) for a, b in zip(g1, g0))


def test_fp8_logits_dE_uses_the_unrounded_activations():
    # E = 0: every logit is 0 whatever the cast, so G = w (1/2 - y) and dE_v = sum_t G_tv A_t
    # with A itself (not fp8(A)); A off the fp8 grid tells the two apart
    T, D, V = 5, 6, 17
    A, _, crow, cids, mask, w = _problem(T, D, V, 22, std=0.37)
    assert not np.array_equal(H.fp8_activations(A), A)
    E = np.zeros((V, D))
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w, A_logits=H.fp8_activations(A))
    assert np.all(dA == 0)
    for v in range(V):
        want = np.zeros(D)
        for t in range(T):
            if mask[t]:
                y = 1.0 if v in set(cids[crow[t]:crow[t + 1]].tolist()) else 0.0
                want += w[t] * (0.5 - y) * A[t]
        np.testing.assert_allclose(dE[v], want, rtol=1e-12, atol=1e-14)


def test_fp8_logits_match_torch_autograd_through_the_cast_input():
    # loss and dA are those of the plain head evaluated at A8 = fp8(A) (torch autograd with A8
    # as the leaf); dE is G^T A
    T, D, V = 7, 16, 45
    A, E, crow, cids, mask, w = _problem(T, D, V, 23, std=1.0)
    A8 = H.fp8_activations(A)
    loss_t, dA_t, _ = _torch_bce(A8, E, crow, cids, mask, w)
    loss = H.bce_loss(A, E, crow, cids, mask, A_logits=A8)
    dA, dE = H.bce_grads(A, E, crow, cids, mask, w, A_logits=A8)
    np.testing.assert_allclose(loss, loss_t, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, dA_t, rtol=1e-10, atol=1e-12)
    X = A8 @ E.T
    G = (w * (mask != 0))[:, None] * (1.0 / (1.0 + np.exp(-X)) - dense_labels(crow, cids, T, V))
    np.testing.assert_allclose(dE, G.T @ A, rtol=1e-12, atol=1e-14)
    # sampled forms agree with the full ones
    lr, dAr = H.bce_rows(A, E, crow, cids, [0, 3], mask, w, A_logits=A8)
    np.testing.assert_allclose(lr, loss[[0, 3]], rtol=1e-13)
    np.testing.assert_allclose(dAr, dA[[0, 3]], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(H.bce_items(A, E, crow, cids, [2, 44], mask, w, A_logits=A8), dE[[2, 44]],
                               rtol=1e-12, atol=1e-15)
