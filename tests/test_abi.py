"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/cutloss.h declares, and rejects bad arguments with the documented
status before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from vocabulary_loss_head_amd import build as build_mod
    if not os.path.exists(build_mod.LIB):
        build_mod.build(verbose=False)
    from vocabulary_loss_head_amd import binding
    return binding


def _declared():
    text = open(os.path.join(ROOT, "include", "cutloss.h")).read()
    return sorted(set(re.findall(r"\b(cutloss_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(B):
    names = _declared()
    assert len(names) >= 10
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def _bce(B, T=64, D=128, V=1000, nnz=256, A=0x10000, E=0x20000, rp=0x30000, ids=0x40000, e_dtype=0):
    return B.BceProblem(T, D, V, A, E, e_dtype, rp, ids, nnz, None, 0)


def _call_fwd(B, p, ws=0x50000, ws_bytes=1 << 40):
    lib = B.lib()
    return lib.cutloss_bce_fwd(ctypes.byref(p) if p is not None else None, ctypes.c_void_p(0x60000),
                               ctypes.c_void_p(ws), ws_bytes, None)


def test_status_strings(B):
    lib = B.lib()
    assert lib.cutloss_status_string(0) == b"ok"
    assert lib.cutloss_status_string(3) == b"workspace too small"
    assert b"gfx950" in lib.cutloss_version()


def test_rejects_bad_arguments_before_launch(B):
    lib = B.lib()
    assert lib.cutloss_bce_fwd(None, None, None, 0, None) == B.ERR_INVALID_ARG
    assert _call_fwd(B, _bce(B, D=100)) == B.ERR_UNSUPPORTED
    assert b"multiple of 64" in lib.cutloss_last_error()
    assert _call_fwd(B, _bce(B, A=0x10001)) == B.ERR_INVALID_ARG
    assert _call_fwd(B, _bce(B, E=0)) == B.ERR_INVALID_ARG
    assert _call_fwd(B, _bce(B, e_dtype=7)) == B.ERR_INVALID_ARG
    assert _call_fwd(B, _bce(B, T=-1)) == B.ERR_INVALID_ARG
    assert _call_fwd(B, _bce(B, nnz=-5)) == B.ERR_INVALID_ARG
    assert _call_fwd(B, _bce(B, ids=0)) == B.ERR_INVALID_ARG
    assert _call_fwd(B, _bce(B), ws_bytes=16) == B.ERR_WORKSPACE
    assert b"workspace too small" in lib.cutloss_last_error()
    assert _call_fwd(B, _bce(B), ws=0x50008) == B.ERR_INVALID_ARG   # misaligned workspace
    # bwd: misaligned output
    p = _bce(B)
    st = lib.cutloss_bce_bwd(ctypes.byref(p), None, ctypes.c_void_p(0x70002), None, None,
                             ctypes.c_void_p(0x50000), 1 << 40, None)
    assert st == B.ERR_INVALID_ARG
    # CE: target must be 8-byte aligned
    c = B.CeProblem(8, 64, 100, 0x10000, 0x20000, 0, 0x30004, -100)
    st = lib.cutloss_ce_fwd(ctypes.byref(c), ctypes.c_void_p(0x60000), ctypes.c_void_p(0x61000),
                            ctypes.c_void_p(0x50000), 1 << 40, None)
    assert st == B.ERR_INVALID_ARG


def test_workspace_size_does_not_grow_with_T_times_V(B):
    a = B.cutloss_bce_workspace_size(_bce(B, T=4096, D=256, V=1_000_000, nnz=32768), B.OP_BWD)
    b = B.cutloss_bce_workspace_size(_bce(B, T=4096, D=256, V=4_000_000, nnz=32768), B.OP_BWD)
    assert a > 0 and a == b
    f = B.cutloss_bce_workspace_size(_bce(B, T=4096, D=256, V=1_000_000, nnz=32768), B.OP_FWD)
    assert 0 < f < a
    assert B.cutloss_bce_workspace_size(_bce(B, D=100), B.OP_FWD) == 0
    # far below the materialized logits (4 T V bytes)
    assert a < 4 * 4096 * 1_000_000 / 50


def test_chunked_workspace_holds_a_fraction_of_the_logits(B):
    # the chunked path keeps one vocabulary chunk's bf16 gradient tile, at most an eighth of
    # the T x V logits whatever T is: the 3M-item FP8 head (T = 128) and the LM head (CE)
    # stay far below even a bf16 T x V tensor (2 T V bytes)
    T, D, V = 128, 768, 3_000_000
    p = B.BceProblem(T, D, V, 0x10000, 0x20000, B.FP8_E4M3, 0x30000, 0x40000, 641, None, -1)
    for op in (B.OP_BWD, B.OP_BWD_SGD, B.OP_BWD_SGD_EX):
        ws = B.cutloss_bce_workspace_size(p, op)
        assert 0 < ws < 2 * T * V / 3, (op, ws)
    T, D, V = 8192, 2304, 256_000
    c = B.CeProblem(T, D, V, 0x10000, 0x20000, B.BF16, 0x30000, -100)
    ws = B.cutloss_ce_workspace_size(c, B.OP_BWD)
    assert 0 < ws < 2 * T * V / 3, ws
    # eight times the vocabulary: the tile reaches its fixed 2 GiB budget, and the workspace
    # falls further behind the logits
    big = B.cutloss_ce_workspace_size(B.CeProblem(T, D, 8 * V, 0x10000, 0x20000, B.BF16, 0x30000, -100), B.OP_BWD)
    assert ws < big < 2 * T * (8 * V) / 8
