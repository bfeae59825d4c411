"""Benchmark of the fused multi-label BCE head (forward + backward in one call).

One step = one cutloss_bce_bwd call with the loss emitted by the same pass: target
canonicalization, the vocabulary-tiled dense softplus sum and dA sweep, the sparse
positive terms, the dE sweep and the row finalization, on the sequential-
recommendation workload T = 4096 (B=16, N=256), D = 256, V = 876,939 (Zipf(1.1)
positives, L = 8, 10% padding rows), inputs resident in HBM.

Prints ONE JSON line. value = counted TFLOP/s with 8*T*V*D FLOPs per step (2TVD forward,
6TVD recompute-backward). The roofline object covers the dominant kernel (timed with
HIP events around its launches inside the timed region); the cpu_baseline object
times the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def _cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline(inp, rows_n=512, items_n=4096):
    """Time the oracle (unchanged) on a bounded sample: loss+dA for `rows_n` rows, dE for `items_n` items."""
    from oracle import head_loss as H
    from oracle.formats import decode_bf16
    from oracle.targets import canonical_csr
    w = inp["workload"]
    A64, E64 = decode_bf16(inp["A"]), decode_bf16(inp["E"])
    crow, cids, _ = canonical_csr(inp["row_ptr"], inp["ids"], inp["mask"], w.V, 0)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(w.T, rows_n, replace=False))
    items = np.sort(rng.choice(w.V, items_n, replace=False))
    t0 = time.perf_counter()
    H.bce_rows(A64, E64, crow, cids, rows, inp["mask"])
    H.bce_items(A64, E64, crow, cids, items, inp["mask"])
    dt = time.perf_counter() - t0
    # counted FLOPs of the sampled share of a step: a row carries its forward (2VD) and dA
    # (2VD); an item carries its recompute (2TD) and dE (2TD)
    flops = rows_n * 4.0 * w.V * w.D + items_n * 4.0 * w.T * w.D
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _cpu_threads(), "kind": "oracle",
            "seconds": dt,
            "sample": f"fp64 oracle: loss+dA for {rows_n} rows (one x_t = E A_t pass each) and dE for "
                      f"{items_n} items (x_v = A E_v each) of the same T={w.T}, D={w.D}, V={w.V} inputs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="seqrec_bce")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the vocabulary-parallel design is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    from vocabulary_loss_head_amd import binding as B
    from workloads import make, workload

    w = workload(args.workload)
    inp = make(w)
    dev = torch.device("cuda:0")
    A = torch.from_numpy(inp["A"].view(np.int16)).to(dev).view(torch.bfloat16)
    E = torch.from_numpy(inp["E"].view(np.int16)).to(dev).view(torch.bfloat16)
    rp = torch.from_numpy(inp["row_ptr"]).to(dev)
    ids = torch.from_numpy(inp["ids"]).to(dev)
    mask = torch.from_numpy(inp["mask"]).to(dev)
    prob = B.bce_problem(A, E, rp, ids, mask, w.pad_id)
    ws = B.workspace(B.cutloss_bce_workspace_size(prob, B.OP_BWD), dev)
    loss = torch.empty(w.T, dtype=torch.float32, device=dev)
    dA = torch.empty(w.T, w.D, dtype=torch.bfloat16, device=dev)
    dE = torch.empty(w.V, w.D, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():
        B.cutloss_bce_bwd(prob, None, dA, dE, loss, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    B.cutloss_profile_read()          # clear
    B.cutloss_profile_enable(True)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    B.cutloss_profile_enable(False)
    phases = B.cutloss_profile_read()
    ms = ev0.elapsed_time(ev1) / args.steps

    T, D, V = w.T, w.D, w.V
    flops = 8.0 * T * V * D
    tflops = flops / (ms * 1e-3) / 1e12
    n_valid = int(inp["mask"].sum())
    phase_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in phases.items()}
    # dominant kernel: the rows sweep (recompute + softplus/sigmoid epilogue + dA) or the
    # cols sweep (recompute + dE); each executes 4 T V D FLOPs per launch
    dom = max(("rows_sweep", "cols_sweep"), key=lambda k: phase_ms[k])
    dom_flops = 4.0 * T * V * D
    achieved = dom_flops / (phase_ms[dom] * 1e-3) / 1e12
    peak_mem = torch.cuda.max_memory_allocated() - base_mem + ws.numel() + A.numel() * 2 + E.numel() * 2 \
        + dA.numel() * 2 + dE.numel() * 2
    rec = {
        "metric": "fused fwd+bwd BCE head TFLOP/s & rows/s at V=876,939; % of bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: A,E ~ N(0,1/sqrt(D)) rounded to bf16; Zipf(1.1) positives; 10% masked rows)",
        "config": {"workload": f"{w.name}: multi-label BCE head T={T} (B=16,N=256) D={D} V={V} L={w.L}",
                   "T": T, "D": D, "V": V, "L": w.L, "mask_frac": w.mask_frac,
                   "call": "cutloss_bce_bwd(loss, dA, dE) = fused forward+backward"},
        "rows_per_s": round(T / (ms * 1e-3), 1),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tflops_valid_rows": round(8.0 * n_valid * V * D / (ms * 1e-3) / 1e12, 2),
        "phase_ms": {k: round(v, 4) for k, v in phase_ms.items()},
        "peak_hbm_bytes": int(peak_mem),
        "logits_fp32_bytes": 4 * T * V,
        "roofline": {"kernel": f"k_sweep_{dom.split('_')[0]}", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
