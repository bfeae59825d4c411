"""Plain float64 definitions of the classifier-head losses and gradients (oracle).

Notation (Cut Binary Cross Entropy, paperpeel, §I-A): activations A[T, D] with
T = B*N rows, item embeddings E[V, D], logits X = A E^T in R^{T x V}.
Upstream weights w_t (the gradient of the caller's reduction with respect to
loss_t; default 1) times the row mask.

BCE (Cut BCE §I-A, multi-label BCE over the entire item vocabulary): for a
valid row t
    loss_t = sum_v -[ y_tv log s(x_tv) + (1 - y_tv) log(1 - s(x_tv)) ]
with s the logistic function, evaluated stably through log s(x) = -softplus(-x)
and log(1 - s(x)) = -softplus(x). Reading: the loss is a per-row sum over V
(no batch reduction inside the op; a caller's mean is a choice of w).
Gradient of L = sum_t w_t loss_t:  G = w (s(X) - Y),  dA = G E,  dE = G^T A.

Cut BCE §I-B ("Fused Direct BCE Formulation") names the exact split of this
loss into a dense background sum_v softplus(x_tv) and a sparse correction
-sum_{p in P_t} x_tp; ``bce_loss_dense_sparse`` writes that form out so the
tests can check the identity against the elementwise definition.

Softmax CE (Cut Your Losses, abeam.tech article, section on splitting the loss
into two needed quantities): loss_t = logsumexp_v(x_tv) - x_{t,y_t}; rows with
target == ignore_index contribute 0. Gradient: G = w (softmax(X) - onehot(y)).

Fused SGD (ELMO, ai.info summary, Key Contributions: classifier gradients
fused with the SGD update so they are never stored; momentum-free SGD with FP8
E4M3 weights): E' = fp8(E - lr dE), nearest-even, saturating; for bfloat16 weights
E' = bf16(E - lr dE), nearest-even.

FP8 logits (ELMO, ai.info summary, Methodology: activations are cast to FP8 only for the
matmul that produces the logits): X = fp8(A) E^T with fp8 the E4M3FN nearest-even saturating
cast; the loss and G come from that X, dA = G E, and dE = G^T A with the unrounded A (the
gradient products are not the logit matmul). ``A_logits`` arguments carry fp8(A).

Sampled forms evaluate the same definitions for chosen rows (one pass
x_t = E A_t each) or chosen items (x_{:,v} = A E_v each); they are exact per
sample and let the tests check full-size problems.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16, decode_fp8_e4m3fn, encode_bf16, encode_fp8_e4m3fn
from .targets import dense_labels


# ----------------------------------------------------------------------------
# scalar functions
# ----------------------------------------------------------------------------

def softplus(x):
    """log(1 + e^x) = max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def bce_elementwise(x, y):
    """-[y log s(x) + (1-y) log(1-s(x))] = y softplus(-x) + (1-y) softplus(x)."""
    return y * softplus(-x) + (1.0 - y) * softplus(x)


def _weights(T, valid, dloss):
    w = np.ones(T, dtype=np.float64) if dloss is None else np.asarray(dloss, dtype=np.float64).copy()
    return w * np.asarray(valid, dtype=np.float64)


def _valid_rows(T, mask):
    return np.ones(T, dtype=bool) if mask is None else np.asarray(mask) != 0


# ----------------------------------------------------------------------------
# BCE, full (materializes X; small shapes)
# ----------------------------------------------------------------------------

def fp8_activations(A):
    """The E4M3FN values of A (nearest-even, saturating): the logit product's FP8 input."""
    return decode_fp8_e4m3fn(encode_fp8_e4m3fn(A))


def bce_loss(A, E, crow, cids, mask=None, A_logits=None):
    """Per-row BCE loss[T] by the elementwise definition."""
    T, V = A.shape[0], E.shape[0]
    X = (A if A_logits is None else A_logits) @ E.T
    Y = dense_labels(crow, cids, T, V)
    loss = bce_elementwise(X, Y).sum(axis=1)
    return np.where(_valid_rows(T, mask), loss, 0.0)


def bce_loss_dense_sparse(A, E, crow, cids, mask=None):
    """Per-row BCE loss[T] as dense background minus sparse correction."""
    T = A.shape[0]
    X = A @ E.T
    dense = softplus(X).sum(axis=1)
    sparse = np.array([X[t, cids[crow[t]:crow[t + 1]]].sum() for t in range(T)])
    return np.where(_valid_rows(T, mask), dense - sparse, 0.0)


def positive_logits(A, E, crow, cids):
    """The sparse correction's terms (Cut BCE §I-B): x_tp = A_t . E_p for every canonical
    pair, one indexed dot product each (X is not formed), and their per-row sums.

    Returns (x_pos [nnz'] in the order of cids, sum_x [T]); rows without positives sum to 0."""
    T = A.shape[0]
    crow = np.asarray(crow, dtype=np.int64)
    cids = np.asarray(cids, dtype=np.int64)
    rows = np.repeat(np.arange(T), np.diff(crow))
    x_pos = np.einsum("ij,ij->i", A[rows], E[cids]) if len(cids) else np.zeros(0)
    sum_x = np.zeros(T, dtype=np.float64)
    for t in range(T):
        sum_x[t] = x_pos[crow[t]:crow[t + 1]].sum()
    return x_pos, sum_x


def bce_grads(A, E, crow, cids, mask=None, dloss=None, A_logits=None):
    """(dA, dE) of L = sum_t w_t loss_t."""
    T, V = A.shape[0], E.shape[0]
    X = (A if A_logits is None else A_logits) @ E.T
    Y = dense_labels(crow, cids, T, V)
    w = _weights(T, _valid_rows(T, mask), dloss)
    G = w[:, None] * (sigmoid(X) - Y)
    return G @ E, G.T @ A


# ----------------------------------------------------------------------------
# BCE, sampled (exact per sampled row / item)
# ----------------------------------------------------------------------------

def bce_rows(A, E, crow, cids, rows, mask=None, dloss=None, A_logits=None):
    """loss[rows] and dA[rows] from x_t = E A_t for each sampled row."""
    T, V = A.shape[0], E.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    X = (A if A_logits is None else A_logits)[rows] @ E.T
    Y = np.zeros_like(X)
    for i, t in enumerate(rows):
        Y[i, cids[crow[t]:crow[t + 1]]] = 1.0
    valid = _valid_rows(T, mask)[rows]
    loss = np.where(valid, bce_elementwise(X, Y).sum(axis=1), 0.0)
    w = _weights(T, _valid_rows(T, mask), dloss)[rows]
    G = w[:, None] * (sigmoid(X) - Y)
    return loss, G @ E


def bce_items(A, E, crow, cids, items, mask=None, dloss=None, A_logits=None):
    """dE[items] from x_{:,v} = A E_v for each sampled item."""
    T = A.shape[0]
    items = np.asarray(items, dtype=np.int64)
    X = (A if A_logits is None else A_logits) @ E[items].T
    Y = np.zeros_like(X)
    col = {int(v): j for j, v in enumerate(items)}
    for t in range(T):
        for v in cids[crow[t]:crow[t + 1]].tolist():
            j = col.get(v)
            if j is not None:
                Y[t, j] = 1.0
    w = _weights(T, _valid_rows(T, mask), dloss)
    G = w[:, None] * (sigmoid(X) - Y)
    return G.T @ A


# ----------------------------------------------------------------------------
# softmax cross-entropy
# ----------------------------------------------------------------------------

def _ce_valid(target, V, ignore_index):
    target = np.asarray(target, dtype=np.int64)
    return (target != ignore_index) & (target >= 0) & (target < V)


def logsumexp_rows(X):
    m = X.max(axis=1)
    return m + np.log(np.exp(X - m[:, None]).sum(axis=1))


def ce_forward(A, E, target, ignore_index=-100):
    """(loss[T], lse[T]); lse is given for every row, loss is 0 on ignored rows."""
    T, V = A.shape[0], E.shape[0]
    X = A @ E.T
    lse = logsumexp_rows(X)
    valid = _ce_valid(target, V, ignore_index)
    tgt = np.where(valid, target, 0)
    loss = np.where(valid, lse - X[np.arange(T), tgt], 0.0)
    return loss, lse


def ce_grads(A, E, target, ignore_index=-100, dloss=None):
    T, V = A.shape[0], E.shape[0]
    X = A @ E.T
    lse = logsumexp_rows(X)
    valid = _ce_valid(target, V, ignore_index)
    w = _weights(T, valid, dloss)
    P = np.exp(X - lse[:, None])
    P[np.arange(T)[valid], np.asarray(target)[valid]] -= 1.0
    G = w[:, None] * P
    return G @ E, G.T @ A


def ce_lse(A, E, rows):
    """lse for the given rows (x_t = E A_t per row)."""
    return logsumexp_rows(A[np.asarray(rows, dtype=np.int64)] @ E.T)


def ce_rows(A, E, target, rows, ignore_index=-100, dloss=None):
    """(loss[rows], lse[rows], dA[rows])."""
    T, V = A.shape[0], E.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    X = A[rows] @ E.T
    lse = logsumexp_rows(X)
    valid_all = _ce_valid(target, V, ignore_index)
    valid = valid_all[rows]
    tgt = np.where(valid, np.asarray(target)[rows], 0)
    loss = np.where(valid, lse - X[np.arange(len(rows)), tgt], 0.0)
    w = _weights(T, valid_all, dloss)[rows]
    P = np.exp(X - lse[:, None])
    idx = np.nonzero(valid)[0]
    P[idx, tgt[idx]] -= 1.0
    return loss, lse, (w[:, None] * P) @ E


def ce_items(A, E, target, items, lse_all, ignore_index=-100, dloss=None):
    """dE[items]; needs lse of every row (``ce_lse`` over all rows)."""
    T, V = A.shape[0], E.shape[0]
    items = np.asarray(items, dtype=np.int64)
    X = A @ E[items].T
    P = np.exp(X - np.asarray(lse_all, dtype=np.float64)[:, None])
    valid = _ce_valid(target, V, ignore_index)
    tgt = np.asarray(target, dtype=np.int64)
    col = {int(v): j for j, v in enumerate(items)}
    for t in np.nonzero(valid)[0]:
        j = col.get(int(tgt[t]))
        if j is not None:
            P[t, j] -= 1.0
    w = _weights(T, valid, dloss)
    return (w[:, None] * P).T @ A


def ce_filter_bounds(A, E, target, eps, ignore_index=-100, dloss=None):
    """Largest change the CE gradient filter can make (Cut Your Losses article, the note on
    skipping the softmax tail below numerical precision): with Q = w softmax(X) (the dense
    part of G), dropping any set of entries with |Q_tv| < eps moves dA_td by at most
    sum_{v: |Q_tv| < eps} |Q_tv| |E_vd| and dE_vd by at most sum_{t: |Q_tv| < eps} |Q_tv| |A_td|.
    Returns (bound_dA [T, D], bound_dE [V, D])."""
    T, V = A.shape[0], E.shape[0]
    X = A @ E.T
    lse = logsumexp_rows(X)
    valid = _ce_valid(target, V, ignore_index)
    w = _weights(T, valid, dloss)
    Q = np.abs(w[:, None] * np.exp(X - lse[:, None]))
    Q = np.where(Q < eps, Q, 0.0)
    return Q @ np.abs(E), Q.T @ np.abs(A)


# ----------------------------------------------------------------------------
# fused SGD on FP8 weights
# ----------------------------------------------------------------------------

def sgd_fp8(E_codes, dE, lr):
    """E' = fp8(E - lr dE) for FP8 E4M3FN codes; dE in float64."""
    return encode_fp8_e4m3fn(decode_fp8_e4m3fn(E_codes) - lr * np.asarray(dE, dtype=np.float64))


def sgd_bf16(E_bits, dE, lr):
    """E' = bf16(E - lr dE) (nearest-even) for bfloat16 bit patterns; dE in float64."""
    return encode_bf16(decode_bf16(E_bits) - lr * np.asarray(dE, dtype=np.float64))


def logits_bytes_fp32(T: int, V: int) -> int:
    """Size of a materialized float32 logit tensor (Cut BCE §I-A)."""
    return 4 * T * V
