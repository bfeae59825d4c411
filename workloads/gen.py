"""Seeded synthetic inputs for the large-vocabulary classifier-head workloads.

This module holds no arithmetic of the loss method. It only draws random
numbers and stores them in the formats the kernels read:

* activations ``A[T, D]`` and embeddings ``E[V, D]`` as bfloat16 bit patterns
  (uint16, round-to-nearest-even from float32 draws), or ``E`` as OCP FP8
  E4M3FN bytes (uint8, nearest with ties to the even code, saturating at 448);
* multi-label positives as CSR (``row_ptr[T+1]``, ``ids[nnz]``, int32) with a
  row mask (uint8, 1 = valid), or one class target per row (int64) for the
  softmax variant, where ``-100`` marks an ignored row.

Every tensor has its own PCG64 stream spawned from ``SeedSequence(seed)``, so
the HIP path and the CPU oracle receive identical bytes.

Workload shapes and distributions follow the pages:
* Cut Binary Cross Entropy (paperpeel), §I-A: sequential-recommendation heads
  with V = 876,939 (876,938 items plus one padding row, ID 0) at local batch
  16 x 256; §III-E: L = 8 next items per position, padded target lists;
  §IV-A: the mini-benchmark draws A, E ~ N(0, I) and uniform targets in [0, V).
  Item popularity is not given on the page; a truncated Zipf(1.1) over item
  IDs 1..V-1 stands in for it.
* ELMO (ai.info summary), Main Findings: a 3-million-label head at batch 128
  with a 768-wide BERT-base encoder, FP8 E4M3 classifier weights.
* Cut Your Losses (abeam.tech article), experiments section: a Gemma-2-2B-like
  LM head (D = 2304, V = 256,000) with one target token per row.
The Yambda, Amazon-3M and LLM corpora are not available; these synthetic
draws of the same shapes stand in for them.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make", "fp8_e4m3fn_values"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "bce" | "ce"
    T: int
    D: int
    V: int
    e_dtype: str         # "bf16" | "fp8"
    a_std: float | None  # None -> 1/sqrt(D)
    e_std: float | None  # None -> 1/sqrt(D)
    targets: str         # "uniform_distinct" | "zipf" | "poisson_distinct" | "uniform_any" | "ce_uniform"
    L: int = 8           # positives per row (fixed-L samplers)
    pad_id: int = 0      # padding item id, -1 = none
    mask_frac: float = 0.0
    ignore_frac: float = 0.0
    lr: float = 0.0
    seed: int = 0

    def std_a(self) -> float:
        return self.a_std if self.a_std is not None else 1.0 / math.sqrt(self.D)

    def std_e(self) -> float:
        return self.e_std if self.e_std is not None else 1.0 / math.sqrt(self.D)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny multi-label head, full oracle
    "tiny_bce": Workload("tiny_bce", "bce", 32, 64, 1000, "bf16", None, None,
                         "uniform_distinct", L=8, pad_id=0, seed=1),
    # sequential-recommendation head at V = 876,939 (the headline workload)
    "seqrec_bce": Workload("seqrec_bce", "bce", 4096, 256, 876939, "bf16", None, None,
                           "zipf", L=8, pad_id=0, mask_frac=0.10, seed=2),
    "seqrec_bce_large": Workload("seqrec_bce_large", "bce", 16384, 512, 876939, "bf16", None, None,
                                 "zipf", L=8, pad_id=0, mask_frac=0.10, seed=3),
    # softmax cross-entropy LM head
    "llm_ce": Workload("llm_ce", "ce", 8192, 2304, 256000, "bf16", None, None,
                       "ce_uniform", L=1, pad_id=-1, ignore_frac=0.05, seed=4),
    # extreme multi-label head, fp8 weights, fused SGD
    "xmc_sgd": Workload("xmc_sgd", "bce", 128, 768, 3000000, "fp8", None, 0.05,
                        "poisson_distinct", L=5, pad_id=-1, lr=0.01, seed=5),
    # the Cut BCE mini-benchmark shape (§IV-A): B = N = 128, V = 100k, D = 128, L = 8,
    # A, E ~ N(0, I), targets uniform in [0, V); a point of comparison with the page's
    # timing, not one of the five configurations
    "cutbce_minibench": Workload("cutbce_minibench", "bce", 16384, 128, 100000, "bf16", 1.0, 1.0,
                                 "uniform_any", L=8, pad_id=-1, seed=6),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.scaled(**overrides) if overrides else w


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def fp8_e4m3fn_values() -> np.ndarray:
    """The 128 non-negative codes 0x00..0x7F of OCP E4M3FN as float64 (0x7F is NaN)."""
    vals = np.empty(128, dtype=np.float64)
    for c in range(128):
        e, m = c >> 3, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = m * 2.0 ** -9
        else:
            vals[c] = (8 + m) * 2.0 ** (e - 10)
    return vals


def _fp8_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN byte: nearest, ties to the even code, |x| > 448 saturates to 448.

    Normal codes (|x| >= 2^-6): round the float32 mantissa to 3 bits (nearest, ties to
    even) by integer arithmetic on the bit pattern, then re-bias the exponent (127 -> 7).
    Subnormal codes (|x| < 2^-6): the code is |x| / 2^-9 rounded to nearest even.
    A negative input sets the sign bit unless it rounds to zero.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(448.0))
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(20)) & np.uint32(1)
    r = (u + np.uint32(0x7FFFF) + lsb) & np.uint32(0xFFF00000)
    e = (r >> np.uint32(23)).astype(np.int32) - 127 + 7
    m = ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    normal = (e << 3) | m
    normal = np.minimum(normal, 0x7E)                       # 464 would round to 480: saturate
    sub = np.rint(a * np.float32(512.0)).astype(np.int32)   # multiples of 2^-9, 0..8
    code = np.where(a >= np.float32(2.0 ** -6), normal, sub).astype(np.uint8)
    neg = np.signbit(x) & (code != 0)
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)


# ----------------------------------------------------------------------------
# samplers
# ----------------------------------------------------------------------------

_CHUNK_ELEMS = 1 << 22


def _normal_matrix(seq: np.random.SeedSequence, rows: int, cols: int, std: float, encode, dtype) -> np.ndarray:
    """rows x cols normals (fp32 draws scaled by std) in chunks of whole rows, each chunk
    with its own spawned stream, encoded by `encode`."""
    out = np.empty((rows, cols), dtype=dtype)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    starts = list(range(0, rows, step))
    seqs = seq.spawn(len(starts))

    def fill(i):
        r0 = starts[i]
        r1 = min(rows, r0 + step)
        g = np.random.Generator(np.random.PCG64(seqs[i]))
        z = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        z *= np.float32(std)
        out[r0:r1] = encode(z)

    with ThreadPoolExecutor(max_workers=16) as ex:
        list(ex.map(fill, range(len(starts))))
    return out


def _normal_bf16(seq: np.random.SeedSequence, rows: int, cols: int, std: float) -> np.ndarray:
    return _normal_matrix(seq, rows, cols, std, _bf16_bits, np.uint16)


def _normal_fp8(seq: np.random.SeedSequence, rows: int, cols: int, std: float) -> np.ndarray:
    return _normal_matrix(seq, rows, cols, std, _fp8_bytes, np.uint8)


def _distinct_rows(draw, T: int, counts: np.ndarray) -> list[np.ndarray]:
    """Per row, keep drawing until `counts[t]` distinct values are seen (draw order kept)."""
    rows = []
    for t in range(T):
        need = int(counts[t])
        got: list[int] = []
        seen: set[int] = set()
        while len(got) < need:
            for v in draw(max(2 * need, 8)):
                v = int(v)
                if v not in seen:
                    seen.add(v)
                    got.append(v)
                    if len(got) == need:
                        break
        rows.append(np.asarray(got, dtype=np.int32))
    return rows


def _zipf_cdf(V: int, s: float) -> np.ndarray:
    k = np.arange(1, V, dtype=np.float64)          # item ids 1..V-1, id = popularity rank
    p = k ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def make(w: Workload, seed: int | None = None, with_dloss: bool = False) -> dict:
    """Draw one batch of inputs for workload `w`.

    Returns a dict of numpy arrays: A (uint16 bf16 bits [T, D]), E (uint16 [V, D]
    or uint8 fp8 [V, D]), and for BCE row_ptr/ids (int32) and mask (uint8 [T]),
    for CE target (int64 [T]); optionally dloss (float32 [T], upstream weights).
    """
    ss = np.random.SeedSequence(w.seed if seed is None else seed)
    s_a, s_e, s_t, s_m, s_w = ss.spawn(5)
    T, D, V = w.T, w.D, w.V
    out: dict = {"workload": w}
    out["A"] = _normal_bf16(s_a, T, D, w.std_a())
    if w.e_dtype == "bf16":
        out["E"] = _normal_bf16(s_e, V, D, w.std_e())
    elif w.e_dtype == "fp8":
        out["E"] = _normal_fp8(s_e, V, D, w.std_e())
    else:
        raise ValueError(w.e_dtype)

    g = np.random.Generator(np.random.PCG64(s_t))
    if w.kind == "ce":
        tgt = g.integers(0, V, size=T, dtype=np.int64)
        n_ign = int(round(w.ignore_frac * T))
        if n_ign:
            gm = np.random.Generator(np.random.PCG64(s_m))
            tgt[gm.permutation(T)[:n_ign]] = -100
        out["target"] = tgt
    else:
        if w.targets == "uniform_distinct":      # L distinct ids in [1, V)
            rows = _distinct_rows(lambda n: g.integers(1, V, size=n), T, np.full(T, w.L))
        elif w.targets == "zipf":                # L distinct Zipf(1.1) ids in [1, V)
            cdf = _zipf_cdf(V, 1.1)
            rows = _distinct_rows(
                lambda n: np.minimum(np.searchsorted(cdf, g.random(n), side="right"), V - 2) + 1,
                T, np.full(T, w.L))
        elif w.targets == "poisson_distinct":    # max(1, Poisson(L)) distinct ids in [0, V)
            counts = np.maximum(1, g.poisson(w.L, size=T))
            rows = _distinct_rows(lambda n: g.integers(0, V, size=n), T, counts)
        elif w.targets == "uniform_any":         # L ids uniform in [0, V), repeats and pad allowed
            rows = [g.integers(0, V, size=w.L).astype(np.int32) for _ in range(T)]
        else:
            raise ValueError(w.targets)
        lens = np.array([len(r) for r in rows], dtype=np.int64)
        row_ptr = np.zeros(T + 1, dtype=np.int32)
        row_ptr[1:] = np.cumsum(lens)
        out["row_ptr"] = row_ptr
        out["ids"] = (np.concatenate(rows).astype(np.int32) if T else np.zeros(0, np.int32))
        mask = np.ones(T, dtype=np.uint8)
        n_mask = int(round(w.mask_frac * T))
        if n_mask:
            gm = np.random.Generator(np.random.PCG64(s_m))
            mask[gm.permutation(T)[:n_mask]] = 0
        out["mask"] = mask
    if with_dloss:
        gw = np.random.Generator(np.random.PCG64(s_w))
        out["dloss"] = gw.uniform(0.5, 1.5, size=T).astype(np.float32)
    return out
