"""Thin ctypes binding of the cutloss C ABI (include/cutloss.h).

Argument marshalling only: every function takes torch tensors that already live on
the GPU, passes their device pointers and the current HIP stream to the library
entry point of the same name, and raises ``CutlossError`` on a non-OK status. No
step of the computation runs here. If the shared library is missing the import of
this module fails loudly: there is no fallback path. The environment variable
CUTLOSS_LIBRARY names another build of the same library to load instead (for
comparing kernel builds).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("CUTLOSS_LIBRARY") or os.path.join(_HERE, "libcutloss.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, FP8_E4M3 = 0, 1
OP_FWD, OP_BWD, OP_BWD_SGD, OP_FWD_METRICS, OP_BWD_SGD_EX = 0, 1, 2, 3, 4
ROUND_NEAREST_EVEN, ROUND_STOCHASTIC = 0, 1


class CutlossError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"cutloss status {status}: {msg}")
        self.status = status


class BceProblem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("D", ctypes.c_int64), ("V", ctypes.c_int64),
        ("A", ctypes.c_void_p), ("E", ctypes.c_void_p), ("e_dtype", ctypes.c_int),
        ("pos_row_ptr", ctypes.c_void_p), ("pos_ids", ctypes.c_void_p), ("nnz", ctypes.c_int64),
        ("row_mask", ctypes.c_void_p), ("pad_id", ctypes.c_int32),
    ]


class CeProblem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("D", ctypes.c_int64), ("V", ctypes.c_int64),
        ("A", ctypes.c_void_p), ("E", ctypes.c_void_p), ("e_dtype", ctypes.c_int),
        ("target", ctypes.c_void_p), ("ignore_index", ctypes.c_int64),
    ]


class SgdOptions(ctypes.Structure):
    _fields_ = [("rounding", ctypes.c_int32), ("seed", ctypes.c_uint64), ("fp8_logits", ctypes.c_int32)]


EXPORTED = [
    "cutloss_bce_workspace_size", "cutloss_ce_workspace_size",
    "cutloss_bce_fwd", "cutloss_bce_fwd_metrics", "cutloss_bce_bwd", "cutloss_bce_bwd_noalloc", "cutloss_bce_bwd_sgd",
    "cutloss_bce_bwd_sgd_ex",
    "cutloss_ce_fwd", "cutloss_ce_bwd", "cutloss_ce_bwd_filtered",
    "cutloss_read_data_errors", "cutloss_bce_canonical_targets", "cutloss_bce_positive_logits",
    "cutloss_profile_enable", "cutloss_profile_read",
    "cutloss_status_string", "cutloss_last_error", "cutloss_version",
]
PHASES = ["targets", "rows_sweep", "finalize_rows", "item_sums", "cols_sweep", "chunk_logits", "chunk_dA",
          "chunk_dE"]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"cutloss HIP library not built: {LIB_PATH} is missing "
                          "(run `python -m vocabulary_loss_head_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sz = ctypes.c_size_t
    st = ctypes.c_int
    pb, pc = ctypes.POINTER(BceProblem), ctypes.POINTER(CeProblem)
    sig = {
        "cutloss_bce_workspace_size": (sz, [pb, ctypes.c_int32]),
        "cutloss_ce_workspace_size": (sz, [pc, ctypes.c_int32]),
        "cutloss_bce_fwd": (st, [pb, P, P, sz, P]),
        "cutloss_bce_fwd_metrics": (st, [pb, P, P, P, sz, P]),
        "cutloss_bce_bwd": (st, [pb, P, P, P, P, P, sz, P]),
        "cutloss_bce_bwd_noalloc": (st, [pb, P, P, P, P, P]),
        "cutloss_bce_bwd_sgd": (st, [pb, P, ctypes.c_float, P, P, P, sz, P]),
        "cutloss_bce_bwd_sgd_ex": (st, [pb, P, ctypes.c_float, ctypes.POINTER(SgdOptions), P, P, P, sz, P]),
        "cutloss_ce_fwd": (st, [pc, P, P, P, sz, P]),
        "cutloss_ce_bwd": (st, [pc, P, P, P, P, P, sz, P]),
        "cutloss_ce_bwd_filtered": (st, [pc, P, P, P, P, ctypes.c_float, P, sz, P]),
        "cutloss_read_data_errors": (st, [P, P, ctypes.POINTER(ctypes.c_int64)]),
        "cutloss_bce_canonical_targets": (st, [pb, P, P, P, P, ctypes.POINTER(ctypes.c_int64), P, sz, P]),
        "cutloss_bce_positive_logits": (st, [pb, P, P, P, sz, P]),
        "cutloss_profile_enable": (st, [ctypes.c_int32]),
        "cutloss_profile_read": (st, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]),
        "cutloss_status_string": (ctypes.c_char_p, [st]),
        "cutloss_last_error": (ctypes.c_char_p, []),
        "cutloss_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != OK:
        raise CutlossError(status, _lib.cutloss_last_error().decode())


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("cutloss takes device tensors")
    if not t.is_contiguous():
        raise ValueError("cutloss takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _e_dtype(E: torch.Tensor) -> int:
    if E.dtype == torch.bfloat16:
        return BF16
    if E.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise ValueError(f"E must be bfloat16 or fp8 e4m3 (uint8 bytes), got {E.dtype}")


def bce_problem(A, E, pos_row_ptr, pos_ids, row_mask=None, pad_id: int = 0) -> BceProblem:
    if A.dtype != torch.bfloat16:
        raise ValueError("A must be bfloat16")
    if pos_row_ptr.dtype != torch.int32 or pos_ids.dtype != torch.int32:
        raise ValueError("pos_row_ptr and pos_ids must be int32")
    if row_mask is not None and row_mask.dtype not in (torch.uint8, torch.bool):
        raise ValueError("row_mask must be uint8")
    T, D = A.shape
    return BceProblem(T, D, E.shape[0], _ptr(A), _ptr(E), _e_dtype(E), _ptr(pos_row_ptr), _ptr(pos_ids),
                      pos_ids.numel(), _ptr(row_mask), pad_id)


def ce_problem(A, E, target, ignore_index: int = -100) -> CeProblem:
    if A.dtype != torch.bfloat16:
        raise ValueError("A must be bfloat16")
    if target.dtype != torch.int64:
        raise ValueError("target must be int64")
    T, D = A.shape
    return CeProblem(T, D, E.shape[0], _ptr(A), _ptr(E), _e_dtype(E), _ptr(target), ignore_index)


def cutloss_bce_workspace_size(problem: BceProblem, op: int) -> int:
    return int(_lib.cutloss_bce_workspace_size(ctypes.byref(problem), op))


def cutloss_ce_workspace_size(problem: CeProblem, op: int) -> int:
    return int(_lib.cutloss_ce_workspace_size(ctypes.byref(problem), op))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A device buffer for the library's scratch space (torch allocations are 512-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def cutloss_bce_fwd(problem: BceProblem, loss, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.cutloss_bce_fwd(ctypes.byref(problem), _ptr(loss), _ptr(ws), ws.numel(), _stream(stream)))


def cutloss_bce_fwd_metrics(problem: BceProblem, loss, counts, ws: torch.Tensor, stream=None) -> None:
    """loss [T] fp32 and counts [T, 4] int32 = (TP, FP, FN, TN) per row."""
    _check(_lib.cutloss_bce_fwd_metrics(ctypes.byref(problem), _ptr(loss), _ptr(counts), _ptr(ws), ws.numel(),
                                        _stream(stream)))


def cutloss_bce_bwd(problem: BceProblem, dloss, dA, dE, loss_out, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.cutloss_bce_bwd(ctypes.byref(problem), _ptr(dloss), _ptr(dA), _ptr(dE), _ptr(loss_out),
                                _ptr(ws), ws.numel(), _stream(stream)))


def cutloss_bce_bwd_noalloc(problem: BceProblem, dloss, dA, dE, loss_out, stream=None) -> None:
    """cutloss_bce_bwd with the library's fixed scratch array instead of a workspace."""
    _check(_lib.cutloss_bce_bwd_noalloc(ctypes.byref(problem), _ptr(dloss), _ptr(dA), _ptr(dE), _ptr(loss_out),
                                        _stream(stream)))


STATIC_SCRATCH_BYTES = 64 << 20


def cutloss_bce_bwd_sgd(problem: BceProblem, dloss, lr: float, dA, loss_out, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.cutloss_bce_bwd_sgd(ctypes.byref(problem), _ptr(dloss), float(lr), _ptr(dA), _ptr(loss_out),
                                    _ptr(ws), ws.numel(), _stream(stream)))


def cutloss_bce_bwd_sgd_ex(problem: BceProblem, dloss, lr: float, dA, loss_out, ws: torch.Tensor, *,
                           stochastic: bool = False, seed: int = 0, fp8_logits: bool = False, stream=None) -> None:
    opt = SgdOptions(ROUND_STOCHASTIC if stochastic else ROUND_NEAREST_EVEN, int(seed) & (2 ** 64 - 1),
                     1 if fp8_logits else 0)
    _check(_lib.cutloss_bce_bwd_sgd_ex(ctypes.byref(problem), _ptr(dloss), float(lr), ctypes.byref(opt), _ptr(dA),
                                       _ptr(loss_out), _ptr(ws), ws.numel(), _stream(stream)))


def cutloss_ce_fwd(problem: CeProblem, loss, lse, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.cutloss_ce_fwd(ctypes.byref(problem), _ptr(loss), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def cutloss_ce_bwd(problem: CeProblem, lse, dloss, dA, dE, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.cutloss_ce_bwd(ctypes.byref(problem), _ptr(lse), _ptr(dloss), _ptr(dA), _ptr(dE),
                               _ptr(ws), ws.numel(), _stream(stream)))


def cutloss_ce_bwd_filtered(problem: CeProblem, lse, dloss, dA, dE, grad_filter_eps: float, ws: torch.Tensor,
                            stream=None) -> None:
    _check(_lib.cutloss_ce_bwd_filtered(ctypes.byref(problem), _ptr(lse), _ptr(dloss), _ptr(dA), _ptr(dE),
                                        float(grad_filter_eps), _ptr(ws), ws.numel(), _stream(stream)))


def cutloss_read_data_errors(ws: torch.Tensor, stream=None) -> int:
    n = ctypes.c_int64(0)
    _check(_lib.cutloss_read_data_errors(_ptr(ws), _stream(stream), ctypes.byref(n)))
    return int(n.value)


def cutloss_bce_canonical_targets(problem: BceProblem, crow, cids, items, rows, ws: torch.Tensor, stream=None) -> int:
    n = ctypes.c_int64(0)
    _check(_lib.cutloss_bce_canonical_targets(ctypes.byref(problem), _ptr(crow), _ptr(cids), _ptr(items), _ptr(rows),
                                              ctypes.byref(n), _ptr(ws), ws.numel(), _stream(stream)))
    return int(n.value)


def cutloss_bce_positive_logits(problem: BceProblem, sum_x, x_pos, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.cutloss_bce_positive_logits(ctypes.byref(problem), _ptr(sum_x), _ptr(x_pos), _ptr(ws), ws.numel(),
                                            _stream(stream)))


def cutloss_profile_enable(enable: bool) -> None:
    _check(_lib.cutloss_profile_enable(1 if enable else 0))


def cutloss_profile_read() -> dict:
    """{phase name: (summed ms, launches)} since the last read (synchronizes)."""
    n = len(PHASES)
    ms = (ctypes.c_float * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(_lib.cutloss_profile_read(ms, cnt, n))
    return {PHASES[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


def cutloss_version() -> str:
    return _lib.cutloss_version().decode()
