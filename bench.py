"""Benchmark of the fused classifier-head losses on one GPU.

Default: one step = one cutloss_bce_bwd call with the loss emitted by the same pass
(fused forward+backward) on the sequential-recommendation head T = 4096 (B=16, N=256),
D = 256, V = 876,939 (Zipf(1.1) positives, L = 8, 10% padding rows), inputs resident in
HBM. It prints ONE JSON line: value = counted TFLOP/s with 8*T*V*D FLOPs per step (2TVD
forward, 6TVD recompute-backward) over `--steps` back-to-back steps timed with nothing else
recorded; a `roofline` object for the dominant kernel, whose launch duration comes from a
separate pass of the same length with the library's HIP events recorded around each kernel
phase on the launch stream; and a `cpu_baseline` object that times the fp64 CPU oracle on a
bounded sample of the same workload.

--workload NAME times another configuration the same way (its fused step: BCE
cutloss_bce_bwd with loss; softmax CE cutloss_ce_fwd + cutloss_ce_bwd; the FP8 XMC head
cutloss_bce_bwd_sgd with loss). --all prints one report line per configuration (not the
benchmark contract line): median, p10 and p90 of 500 (or, for the two heaviest heads, 100)
back-to-back forward calls and fused steps (the Cut BCE mini-benchmark's steady-state
protocol, §IV-A), counted rates over all rows and over valid rows, fractions of the bf16
MFMA peak (and of the HBM peak for the FP8 head), peak HBM use against the materialized
logits, per-phase times, the separately measured options, and the oracle's CPU time with
the full-size time extrapolated. --all --only --workload NAME reports one configuration.

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
    """Threads the oracle's BLAS actually runs with."""
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def cpu_baseline(inp, rows_n=512, items_n=4096, full=False):
    """Time the oracle (unchanged) on a bounded sample of the same inputs: loss+dA for
    `rows_n` rows (one x_t = E A_t pass each) and dE for `items_n` items (x_v = A E_v each;
    for softmax CE after the logsumexp of every row, whose time is counted with the rows).
    The rate is the metric's counted FLOPs of that share of a step (a row carries 2VD
    forward + 2VD dA, an item 2TD recompute + 2TD dE) per second; the full-size time
    t_row * T + t_item * V is extrapolated from the two per-sample times. full=True runs
    the whole oracle instead (small heads)."""
    from oracle import head_loss as H
    from oracle.formats import decode_bf16, decode_fp8_e4m3fn
    from oracle.targets import canonical_csr
    w = inp["workload"]
    A64 = decode_bf16(inp["A"])
    E64 = decode_bf16(inp["E"]) if inp["E"].dtype == np.uint16 else decode_fp8_e4m3fn(inp["E"])
    rec = {"unit": "TFLOP/s", "cores": _cpu_threads(), "host_cpu_count": os.cpu_count(), "kind": "oracle"}
    if full:
        t0 = time.perf_counter()
        if w.kind == "bce":
            crow, cids, _ = canonical_csr(inp["row_ptr"], inp["ids"], inp["mask"], w.V, w.pad_id)
            H.bce_loss(A64, E64, crow, cids, inp["mask"])
            H.bce_grads(A64, E64, crow, cids, inp["mask"])
        else:
            H.ce_forward(A64, E64, inp["target"])
            H.ce_grads(A64, E64, inp["target"])
        dt = time.perf_counter() - t0
        rec.update({"value": 8.0 * w.T * w.V * w.D / dt / 1e12, "seconds": round(dt, 4),
                    "full_size_seconds": round(dt, 4),
                    "sample": f"fp64 oracle, whole fwd+bwd (logits materialized) of T={w.T}, D={w.D}, V={w.V}"})
        return rec
    rng = np.random.default_rng(0)
    rows_n = min(rows_n, w.T)
    items_n = min(items_n, w.V)
    rows = np.sort(rng.choice(w.T, rows_n, replace=False))
    items = np.sort(rng.choice(w.V, items_n, replace=False))
    if w.kind == "bce":
        crow, cids, _ = canonical_csr(inp["row_ptr"], inp["ids"], inp["mask"], w.V, w.pad_id)
        t0 = time.perf_counter()
        H.bce_rows(A64, E64, crow, cids, rows, inp["mask"])
        t1 = time.perf_counter()
        H.bce_items(A64, E64, crow, cids, items, inp["mask"])
        t2 = time.perf_counter()
        t_row, t_item = (t1 - t0) / rows_n, (t2 - t1) / items_n
    else:
        t0 = time.perf_counter()
        H.ce_rows(A64, E64, inp["target"], rows)
        t1 = time.perf_counter()
        # dE of an item needs the logsumexp of every row: the oracle's own values, stored by
        # tests/golden/make_llm_ce_lse.py for the LM head (its time is the rows' forward
        # pass, already in t_row), else computed here and counted with the rows
        lse_all = None
        gold = os.path.join(ROOT, "tests", "golden", f"{w.name}_lse.npy")
        if os.path.exists(gold):
            lse_all = np.load(gold)
            if lse_all.shape != (w.T,):
                lse_all = None
        t_lse = 0.0
        if lse_all is None:
            lse_all = H.ce_lse(A64, E64, np.arange(w.T))
            t_lse = time.perf_counter() - t1
        t2 = time.perf_counter()
        H.ce_items(A64, E64, inp["target"], items, lse_all)
        t3 = time.perf_counter()
        t_row, t_item = (t1 - t0) / rows_n + t_lse / w.T, (t3 - t2) / items_n
        t2 = t3
    dt = t2 - t0
    flops = rows_n * 4.0 * w.V * w.D + items_n * 4.0 * w.T * w.D
    rec.update({"value": flops / dt / 1e12, "seconds": round(dt, 3),
                "extrapolated_full_size_seconds": round(t_row * w.T + t_item * w.V, 1),
                "sample": f"fp64 oracle: loss+dA for {rows_n} rows (one x_t = E A_t pass each) and dE for "
                          f"{items_n} items (x_v = A E_v each) of the same T={w.T}, D={w.D}, V={w.V} inputs; "
                          f"full size extrapolated as t_row*T + t_item*V"})
    return rec


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
    """Mean ms per call of `steps` back-to-back calls after `warmup` untimed ones, bracketed
    by device synchronizations. With profile=True the library's per-phase HIP events are
    recorded (a separate pass from the timed contract line) and returned as
    {phase: (ms per step, launches per step)}."""
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
        phases = {k: (v[0] / steps, v[1] / steps) for k, v in B.cutloss_profile_read().items() if v[1]}
    return ev0.elapsed_time(ev1) / steps, phases


def time_per_call(fn, n, warmup):
    """Per-call device times of n back-to-back calls (a HIP event on the calling stream
    between consecutive calls), after `warmup` untimed calls: median, p10, p90, mean (ms)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record()
    for i in range(n):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n)])
    return {"median": round(float(np.median(t)), 4), "p10": round(float(np.percentile(t, 10)), 4),
            "p90": round(float(np.percentile(t, 90)), 4), "mean": round(float(t.mean()), 4), "calls": n}


def e_bytes(w):
    return w.V * w.D * (1 if w.e_dtype == "fp8" else 2)


def _load(name):
    import torch
    from workloads import make, workload
    inp = make(workload(name))
    h = Head(inp)
    torch.cuda.synchronize()
    return inp, h


def _dominant_sweep(phases):
    # dominant kernel phase of the fused sweeps (D <= 256): one launch per step each;
    # each sweep executes 4TVD per launch (logit recompute + dA or dE)
    return max(("rows_sweep", "cols_sweep"), key=lambda k: phases.get(k, (0.0, 0))[0])


def record(name, steps, warmup, with_cpu):
    """The contract line: `steps` fused steps timed with nothing else recorded, then a
    separate pass of the same length with the library's phase events for the roofline."""
    import torch
    inp, h = _load(name)
    w = h.w
    torch.cuda.reset_peak_memory_stats()
    ms, _ = time_calls(h.step, steps, warmup, profile=False)
    peak = torch.cuda.max_memory_allocated()
    _, phases = time_calls(h.step, steps, 1, profile=True)
    T, D, V = w.T, w.D, w.V
    tflops = 8.0 * T * V * D / (ms * 1e-3) / 1e12
    n_valid = int(inp["mask"].sum()) if "mask" in inp else int((inp["target"] != -100).sum())
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
        dom = _dominant_sweep(phases)
        achieved = 4.0 * T * V * D / (phases[dom][0] / phases[dom][1] * 1e-3) / 1e12
        kname = f"k_{dom.split('_')[0]}2"
        rec["roofline"] = {"kernel": f"{kname} (fused {dom.replace('_', ' ')})", "bound": "mfma",
                           "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(kname)}
    if w.lr > 0:
        rec["e_traffic_GBps"] = round(2 * e_bytes(w) / (ms * 1e-3) / 1e9, 1)
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(inp)
    return rec, h


# calls per timed configuration, after the Cut BCE mini-benchmark's 500 steady-state
# iterations (§IV-A); the two heaviest heads take 100
CALLS = {"tiny_bce": 500, "seqrec_bce": 500, "seqrec_bce_large": 100, "llm_ce": 100, "xmc_sgd": 500}


def config_record(name, calls=None, with_cpu=True):
    """One report line per configuration: forward and fused-step call statistics, counted
    rates over all rows and over valid rows, fractions of peak, peak HBM use against the
    materialized logits, per-phase times from a separate profiled pass, the separately
    measured options, and the oracle's CPU time."""
    import torch
    inp, h = _load(name)
    w = h.w
    T, D, V = w.T, w.D, w.V
    n = calls or CALLS.get(name, 500)
    n_valid = int(inp["mask"].sum()) if "mask" in inp else int((inp["target"] != -100).sum())
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    step = time_per_call(h.step, n, 10)
    peak = torch.cuda.max_memory_allocated()
    fwd = time_per_call(h.fwd, n, 10)
    _, phases = time_calls(h.step, min(n, 50), 2, profile=True)
    sm, fm = step["median"] * 1e-3, fwd["median"] * 1e-3
    rec = {
        "workload": name, "kind": w.kind, "T": T, "D": D, "V": V, "e_dtype": w.e_dtype, "valid_rows": n_valid,
        "call": h.call_name(),
        "step_ms": step, "fwd_ms": fwd,
        "rows_per_s": round(T / sm, 1),
        "step_tflops_counted_8TVD": round(8.0 * T * V * D / sm / 1e12, 2),
        "step_tflops_valid_rows": round(8.0 * n_valid * V * D / sm / 1e12, 2),
        "fwd_tflops_counted_2TVD": round(2.0 * T * V * D / fm / 1e12, 2),
        "fwd_tflops_valid_rows": round(2.0 * n_valid * V * D / fm / 1e12, 2),
        "step_pct_bf16_peak": round(100.0 * 8.0 * T * V * D / sm / 1e12 / PEAK_BF16_TFLOPS, 2),
        "fwd_pct_bf16_peak": round(100.0 * 2.0 * T * V * D / fm / 1e12 / PEAK_BF16_TFLOPS, 2),
        "input_bytes_resident": int(base),
        "peak_hbm_bytes": int(peak),
        "workspace_bytes": h.ws_bytes,
        "logits_fp32_bytes": 4 * T * V,
        "phase_ms_per_step": {k: round(v[0], 4) for k, v in phases.items()},
        "phase_launches_per_step": {k: round(v[1], 2) for k, v in phases.items()},
    }
    if w.e_dtype == "fp8":
        # E streaming dominates at T = 128: the forward reads E once; the SGD step reads it
        # at least once and writes it once (two sweeps over E read it twice)
        eb = e_bytes(w)
        rec["fwd_e_read_GBps"] = round(eb / fm / 1e9, 1)
        rec["fwd_pct_hbm_peak"] = round(100.0 * eb / fm / 1e9 / PEAK_HBM_GBS, 2)
        rec["step_e_GBps_single_pass_count"] = round(2 * eb / sm / 1e9, 1)
        rec["step_e_GBps_two_sweep_count"] = round(3 * eb / sm / 1e9, 1)
        rec["step_pct_hbm_peak_two_sweep_count"] = round(100.0 * 3 * eb / sm / 1e9 / PEAK_HBM_GBS, 2)
    opts = {}
    m = max(20, n // 5)
    if w.kind == "bce":
        opts["fwd_cut_metrics_ms"] = time_per_call(h.fwd_metrics, m, 3)
        if h.sgd:
            opts["step_sgd_stochastic_rounding_ms"] = time_per_call(lambda: h.step_sgd_ex(stochastic=True), m, 3)
            opts["step_sgd_fp8_logits_ms"] = time_per_call(lambda: h.step_sgd_ex(fp8_logits=True), m, 3)
            opts["step_sgd_fp8_logits_stochastic_rounding_ms"] = time_per_call(
                lambda: h.step_sgd_ex(stochastic=True, fp8_logits=True), m, 3)
    else:
        opts["step_grad_filter_2^-12_ms"] = time_per_call(h.step_grad_filter, m, 3)
    rec["options"] = opts
    del h
    torch.cuda.empty_cache()
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(inp, full=(name == "tiny_bce"))
    return rec


def report_all(names, with_cpu):
    for name in names:
        print(json.dumps(config_record(name, with_cpu=with_cpu)), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="seqrec_bce", choices=ALL + ["cutbce_minibench"])
    ap.add_argument("--all", action="store_true", help="one report line per configuration")
    ap.add_argument("--only", action="store_true", help="with --all: only the --workload configuration")
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
        report_all(ALL if args.workload == "seqrec_bce" and not args.only else [args.workload],
                   with_cpu=not args.no_cpu_baseline)
        return
    rec, _ = record(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu_baseline)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
