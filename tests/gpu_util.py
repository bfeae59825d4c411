"""Helpers shared by the GPU parity tests: device upload of the seeded inputs, calls
through the C-ABI binding, and the comparison rules.

Tolerances (stated for the whole suite): per-row loss relative error <= 1e-3;
dA and dE max-abs error <= 2e-2 * max|ref| over the compared set and cosine
similarity >= 0.9999; canonical positive sets and masks bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.formats import decode_bf16, decode_fp8_e4m3fn
from oracle.targets import canonical_csr

LOSS_RTOL = 1e-3
GRAD_ATOL_FRAC = 2e-2
GRAD_COS = 0.9999


def dev():
    return torch.device("cuda:0")


def upload(inp: dict) -> dict:
    d = dev()
    out = {"A": torch.from_numpy(inp["A"].view(np.int16)).to(d).view(torch.bfloat16)}
    E = inp["E"]
    if E.dtype == np.uint16:
        out["E"] = torch.from_numpy(E.view(np.int16)).to(d).view(torch.bfloat16)
    else:
        out["E"] = torch.from_numpy(E).to(d)
    for k in ("row_ptr", "ids", "mask", "target", "dloss"):
        if k in inp:
            out[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(d)
    return out


def decode_inputs(inp: dict):
    A = decode_bf16(inp["A"])
    E = decode_bf16(inp["E"]) if inp["E"].dtype == np.uint16 else decode_fp8_e4m3fn(inp["E"])
    return A, E


def canonical(inp: dict, V: int, pad_id: int):
    return canonical_csr(inp["row_ptr"], inp["ids"], inp.get("mask"), V, pad_id)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return decode_bf16(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def check_loss(got, ref, rtol=LOSS_RTOL, what="loss"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = rtol * np.abs(ref) + 1e-30
    bad = np.nonzero(err > bound)[0]
    assert len(bad) == 0, f"{what}: {len(bad)} rows out of tolerance, first {bad[:5]}: got {got[bad[:5]]} ref {ref[bad[:5]]}"


def grad_stats(got, ref):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    mx = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref).max() if ref.size else 0.0
    ng, nr = np.linalg.norm(got), np.linalg.norm(ref)
    cos = float(got @ ref / (ng * nr)) if ng > 0 and nr > 0 else (1.0 if ng == nr else 0.0)
    return err, mx, cos


def check_grad(got, ref, what="grad", atol_frac=GRAD_ATOL_FRAC, cos_min=GRAD_COS):
    err, mx, cos = grad_stats(got, ref)
    if mx == 0.0:
        assert err == 0.0, f"{what}: reference is zero, max |got| = {err}"
        return
    assert err <= atol_frac * mx, f"{what}: max abs err {err:.3e} > {atol_frac} * {mx:.3e}"
    assert cos >= cos_min, f"{what}: cosine {cos:.7f} < {cos_min}"


def run_bce(B, g: dict, pad_id: int, want_loss=True, want_dA=True, want_dE=True, dloss=None, fused_loss=True):
    """Forward, then backward (with the loss emitted by the backward pass too)."""
    A, E = g["A"], g["E"]
    T, D = A.shape
    V = E.shape[0]
    prob = B.bce_problem(A, E, g["row_ptr"], g["ids"], g.get("mask"), pad_id)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD), A.device)
    out = {}
    if want_loss:
        loss = torch.empty(T, dtype=torch.float32, device=A.device)
        B.cutloss_bce_fwd(prob, loss, ws)
        out["loss"] = loss
    dA = torch.empty(T, D, dtype=torch.bfloat16, device=A.device) if want_dA else None
    dE = torch.empty(V, D, dtype=torch.bfloat16, device=A.device) if want_dE else None
    floss = torch.empty(T, dtype=torch.float32, device=A.device) if fused_loss else None
    if want_dA or want_dE or fused_loss:
        B.cutloss_bce_bwd(prob, dloss, dA, dE, floss, ws)
    torch.cuda.synchronize()
    out["dA"], out["dE"], out["floss"] = dA, dE, floss
    out["n_err"] = B.cutloss_read_data_errors(ws)
    return out


def run_ce(B, g: dict, ignore_index=-100, dloss=None, want_dA=True, want_dE=True):
    A, E = g["A"], g["E"]
    T, D = A.shape
    V = E.shape[0]
    prob = B.ce_problem(A, E, g["target"], ignore_index)
    ws = B.workspace(max(B.cutloss_ce_workspace_size(prob, B.OP_BWD), B.cutloss_ce_workspace_size(prob, B.OP_FWD)), A.device)
    loss = torch.empty(T, dtype=torch.float32, device=A.device)
    lse = torch.empty(T, dtype=torch.float32, device=A.device)
    B.cutloss_ce_fwd(prob, loss, lse, ws)
    dA = torch.empty(T, D, dtype=torch.bfloat16, device=A.device) if want_dA else None
    dE = torch.empty(V, D, dtype=torch.bfloat16, device=A.device) if want_dE else None
    if want_dA or want_dE:
        B.cutloss_ce_bwd(prob, lse, dloss, dA, dE, ws)
    torch.cuda.synchronize()
    return {"loss": loss, "lse": lse, "dA": dA, "dE": dE, "n_err": B.cutloss_read_data_errors(ws)}
