"""Benchmark of the fused classifier-head losses on one GPU.

Default: one step = one cutloss_bce_bwd call with the loss emitted by the same pass
(fused forward+backward) on the sequential-recommendation head T = 4096 (B=16, N=256),
D = 256, V = 876,939 (Zipf(1.1) positives, L = 8, 10% padding rows), inputs resident in
HBM. It prints ONE JSON line: value = counted TFLOP/s with 8*T*V*D FLOPs per step (2TVD
forward, 6TVD recompute-backward), a `roofline` object for the dominant kernel (HIP
events recorded by the library around its launches, on the launch stream) and a
`cpu_baseline` object that times the fp64 CPU oracle on a bounded sample of the same
workload.

--workload NAME times another configuration the same way (its fused step: BCE
cutloss_bce_bwd with loss; softmax CE cutloss_ce_fwd + cutloss_ce_bwd; the FP8 XMC head
cutloss_bce_bwd_sgd with loss). --all prints one JSON line per configuration with the
forward-only and fused-step timings (a report, not the benchmark contract line).

roofline.traffic is the HBM byte count per launch of the dominant kernel measured with
rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each scaled by the factor a plain copy of
known size reads on the same counter), stored in profiles/ with the SHA-256 of the
kernel sources it was taken on; it is null when those sources have changed since.
--copy-calibration BYTES runs only that plain copy (torch's device copy kernel), for the
counter runs.
"""
from __future__ import annotations

import argparse
import hashlib
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
METRIC = "fused fwd+bwd BCE head TFLOP/s & rows/s at V=876,939; % of bf16 MFMA peak"
ALL = ["tiny_bce", "seqrec_bce", "seqrec_bce_large", "llm_ce", "xmc_sgd"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "seqrec_bce_sweeps_hbm_traffic.json")
SWEEP_SOURCES = ["vocabulary_loss_head_amd/csrc/sweep2.hip", "vocabulary_loss_head_amd/csrc/common.h"]


def sweep_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in SWEEP_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the stored counter summary, or None when it is
    missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sweep_sources_sha256():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_calibration(nbytes: int, reps: int = 5) -> None:
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n, "reps": reps}), flush=True)


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
    """Time the oracle (unchanged) on a bounded sample: loss+dA for `rows_n` rows and, for
    the multi-label heads, dE for `items_n` items. The rate is counted FLOPs of that
    sampled share of a step per second (a row carries 2VD forward + 2VD dA, an item 2TD
    recompute + 2TD dE)."""
    from oracle import head_loss as H
    from oracle.formats import decode_bf16, decode_fp8_e4m3fn
    from oracle.targets import canonical_csr
    w = inp["workload"]
    A64 = decode_bf16(inp["A"])
    E64 = decode_bf16(inp["E"]) if inp["E"].dtype == np.uint16 else decode_fp8_e4m3fn(inp["E"])
    rng = np.random.default_rng(0)
    rows_n = min(rows_n, w.T)
    items_n = min(items_n, w.V) if w.kind == "bce" else 0
    rows = np.sort(rng.choice(w.T, rows_n, replace=False))
    t0 = time.perf_counter()
    if w.kind == "bce":
        crow, cids, _ = canonical_csr(inp["row_ptr"], inp["ids"], inp["mask"], w.V, w.pad_id)
        H.bce_rows(A64, E64, crow, cids, rows, inp["mask"])
        items = np.sort(rng.choice(w.V, items_n, replace=False))
        H.bce_items(A64, E64, crow, cids, items, inp["mask"])
    else:
        H.ce_rows(A64, E64, inp["target"], rows)
    dt = time.perf_counter() - t0
    flops = rows_n * 4.0 * w.V * w.D + items_n * 4.0 * w.T * w.D
    what = f"loss+dA for {rows_n} rows (one x_t = E A_t pass each)"
    if items_n:
        what += f" and dE for {items_n} items (x_v = A E_v each)"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _cpu_threads(), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"fp64 oracle: {what} of the same T={w.T}, D={w.D}, V={w.V} inputs"}


class Head:
    """Device inputs, outputs and workspace of one workload, and its step callables."""

    def __init__(self, inp):
        import torch
        from vocabulary_loss_head_amd import binding as B
        self.B = B
        self.w = w = inp["workload"]
        dev = torch.device("cuda:0")
        self.A = torch.from_numpy(inp["A"].view(np.int16)).to(dev).view(torch.bfloat16)
        if inp["E"].dtype == np.uint16:
            self.E = torch.from_numpy(inp["E"].view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            self.E = torch.from_numpy(inp["E"]).to(dev)
        T, D, V = w.T, w.D, w.V
        self.loss = torch.empty(T, dtype=torch.float32, device=dev)
        self.dA = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
        if w.kind == "ce":
            self.target = torch.from_numpy(inp["target"]).to(dev)
            self.prob = B.ce_problem(self.A, self.E, self.target, -100)
            self.lse = torch.empty(T, dtype=torch.float32, device=dev)
            self.dE = torch.empty(V, D, dtype=torch.bfloat16, device=dev)
            nb = max(B.cutloss_ce_workspace_size(self.prob, B.OP_BWD), B.cutloss_ce_workspace_size(self.prob, B.OP_FWD))
        else:
            self.rp = torch.from_numpy(inp["row_ptr"]).to(dev)
            self.ids = torch.from_numpy(inp["ids"]).to(dev)
            self.mask = torch.from_numpy(inp["mask"]).to(dev)
            self.prob = B.bce_problem(self.A, self.E, self.rp, self.ids, self.mask, w.pad_id)
            self.sgd = w.lr > 0
            self.dE = None if self.sgd else torch.empty(V, D, dtype=torch.bfloat16, device=dev)
            op = B.OP_BWD_SGD if self.sgd else B.OP_BWD
            nb = B.cutloss_bce_workspace_size(self.prob, op)
        self.ws = B.workspace(nb, dev)
        self.ws_bytes = int(nb)

    def fwd_metrics(self):
        """BCE forward with the Cut Metrics counts (a separately measured option)."""
        import torch
        B = self.B
        if getattr(self, "mws", None) is None:
            self.mws = B.workspace(B.cutloss_bce_workspace_size(self.prob, B.OP_FWD_METRICS), self.A.device)
            self.counts = torch.empty(self.w.T, 4, dtype=torch.int32, device=self.A.device)
        B.cutloss_bce_fwd_metrics(self.prob, self.loss, self.counts, self.mws)

    def fwd(self):
        B = self.B
        if self.w.kind == "ce":
            B.cutloss_ce_fwd(self.prob, self.loss, self.lse, self.ws)
        else:
            B.cutloss_bce_fwd(self.prob, self.loss, self.ws)

    def step(self):
        """One fused forward+backward pass (the benchmark step)."""
        B = self.B
        if self.w.kind == "ce":
            B.cutloss_ce_fwd(self.prob, self.loss, self.lse, self.ws)
            B.cutloss_ce_bwd(self.prob, self.lse, None, self.dA, self.dE, self.ws)
        elif self.sgd:
            B.cutloss_bce_bwd_sgd(self.prob, None, self.w.lr, self.dA, self.loss, self.ws)
        else:
            B.cutloss_bce_bwd(self.prob, None, self.dA, self.dE, self.loss, self.ws)

    def step_grad_filter(self, eps=2.0 ** -12):
        """The CE step with the gradient filter on (a separately measured option)."""
        B = self.B
        B.cutloss_ce_fwd(self.prob, self.loss, self.lse, self.ws)
        B.cutloss_ce_bwd_filtered(self.prob, self.lse, None, self.dA, self.dE, eps, self.ws)

    def step_sgd_ex(self, stochastic=False, fp8_logits=False):
        """The SGD step with ELMO's options (separately measured): stochastic rounding of E
        (a new seed every call) and/or FP8 activations for the logit product."""
        B = self.B
        if getattr(self, "exws", None) is None:
            self.exws = B.workspace(B.cutloss_bce_workspace_size(self.prob, B.OP_BWD_SGD_EX), self.A.device)
            self.sr_seed = 0
        self.sr_seed += 1
        B.cutloss_bce_bwd_sgd_ex(self.prob, None, self.w.lr, self.dA, self.loss, self.exws, stochastic=stochastic,
                                 seed=self.sr_seed, fp8_logits=fp8_logits)

    def call_name(self):
        if self.w.kind == "ce":
            return "cutloss_ce_fwd(loss, lse) + cutloss_ce_bwd(dA, dE)"
        if self.sgd:
            return "cutloss_bce_bwd_sgd(lr, dA, loss): fused forward+backward, E updated in place"
        return "cutloss_bce_bwd(loss, dA, dE) = fused forward+backward"


def time_calls(fn, steps, warmup, profile=False):
    import torch
    from vocabulary_loss_head_amd import binding as B
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if profile:
        B.cutloss_profile_read()
        B.cutloss_profile_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    phases = {}
    if profile:
        B.cutloss_profile_enable(False)
        # {phase: (ms per step, launches per step)}
        phases = {k: (v[0] / steps, v[1] / steps) for k, v in B.cutloss_profile_read().items() if v[1]}
    return ev0.elapsed_time(ev1) / steps, phases


def e_bytes(w):
    return w.V * w.D * (1 if w.e_dtype == "fp8" else 2)


def record(name, steps, warmup, with_cpu):
    import torch
    from workloads import make, workload
    w = workload(name)
    inp = make(w)
    h = Head(inp)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    ms, phases = time_calls(h.step, steps, warmup, profile=True)
    peak = torch.cuda.max_memory_allocated()
    T, D, V = w.T, w.D, w.V
    tflops = 8.0 * T * V * D / (ms * 1e-3) / 1e12
    n_valid = int(inp["mask"].sum()) if "mask" in inp else int((inp["target"] != -100).sum())
    # dominant kernel phase of the fused sweeps (D <= 256): one launch per step each;
    # the rows sweep executes 4TVD per launch (logit recompute + dA)
    dom = max(("rows_sweep", "cols_sweep"), key=lambda k: phases.get(k, (0.0, 0))[0])
    rec = {
        "metric": METRIC if name == "seqrec_bce" else f"{name}: fused fwd+bwd TFLOP/s (8TVD counted)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.e_dtype == "bf16" else "bf16 A x fp8 E (widened to bf16)",
        "data": "synthetic (seeded; A,E ~ N(0, std) rounded to the storage format)",
        "config": {"workload": f"{name}: {'softmax CE' if w.kind == 'ce' else 'multi-label BCE'} head "
                               f"T={T} D={D} V={V}", "T": T, "D": D, "V": V, "call": h.call_name()},
        "rows_per_s": round(T / (ms * 1e-3), 1),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tflops_valid_rows": round(8.0 * n_valid * V * D / (ms * 1e-3) / 1e12, 2),
        "phase_ms": {k: round(v[0], 4) for k, v in phases.items()},
        "phase_launches": {k: round(v[1], 2) for k, v in phases.items()},
        "peak_hbm_bytes": int(peak),
        "workspace_bytes": h.ws_bytes,
        "logits_fp32_bytes": 4 * T * V,
    }
    if name == "seqrec_bce":
        dom_flops = 4.0 * T * V * D
        achieved = dom_flops / (phases[dom][0] / phases[dom][1] * 1e-3) / 1e12
        kname = f"k_{dom.split('_')[0]}2"
        rec["roofline"] = {"kernel": f"{kname} (fused {dom.replace('_', ' ')})", "bound": "mfma",
                           "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(kname)}
    if w.lr > 0:
        # fused SGD step: E is read and written once at the least
        rec["e_traffic_GBps"] = round(2 * e_bytes(w) / (ms * 1e-3) / 1e9, 1)
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(inp)
    return rec, h


def report_all(steps, warmup):
    import torch
    for name in ALL:
        rec, h = record(name, steps, warmup, with_cpu=False)
        fwd_ms, fwd_phases = time_calls(h.fwd, steps, warmup)
        w = h.w
        rec["fwd_ms"] = round(fwd_ms, 4)
        rec["fwd_tflops"] = round(2.0 * w.T * w.V * w.D / (fwd_ms * 1e-3) / 1e12, 2)
        rec["fwd_pct_bf16_peak"] = round(100.0 * rec["fwd_tflops"] / PEAK_BF16_TFLOPS, 2)
        rec["fwd_e_read_GBps"] = round(e_bytes(w) / (fwd_ms * 1e-3) / 1e9, 1)
        if w.kind == "bce":
            m_ms, _ = time_calls(h.fwd_metrics, steps, warmup)
            rec["fwd_cut_metrics_ms"] = round(m_ms, 4)
            if h.sgd:
                s_ms, _ = time_calls(lambda: h.step_sgd_ex(stochastic=True), steps, warmup)
                rec["step_sgd_stochastic_rounding_ms"] = round(s_ms, 4)
                f_ms, _ = time_calls(lambda: h.step_sgd_ex(fp8_logits=True), steps, warmup)
                rec["step_sgd_fp8_logits_ms"] = round(f_ms, 4)
                b_ms, _ = time_calls(lambda: h.step_sgd_ex(stochastic=True, fp8_logits=True), steps, warmup)
                rec["step_sgd_fp8_logits_stochastic_rounding_ms"] = round(b_ms, 4)
        else:
            f_ms, _ = time_calls(h.step_grad_filter, steps, warmup)
            rec["step_grad_filter_2^-12_ms"] = round(f_ms, 4)
        print(json.dumps(rec), flush=True)
        del h
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="seqrec_bce", choices=ALL)
    ap.add_argument("--all", action="store_true", help="one report line per configuration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the vocabulary-parallel form is designed but not built)", file=sys.stderr)
        sys.exit(2)
    if args.all:
        report_all(args.steps, args.warmup)
        return
    rec, _ = record(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu_baseline)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
