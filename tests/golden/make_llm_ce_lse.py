"""Write tests/golden/llm_ce_lse.npy: the fp64 oracle's logsumexp of every row of the
softmax-CE workload `llm_ce` (T = 8192, D = 2304, V = 256,000; seeded inputs from
workloads.make). The full-size GPU test needs it to check dE on sampled items, since
softmax probabilities of an item involve the normalizer of every row.

Calls only the oracle (oracle.head_loss.ce_lse) and the seeded input generator.
Run from the repository root: python tests/golden/make_llm_ce_lse.py (a few minutes).
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.formats import decode_bf16  # noqa: E402
from oracle.head_loss import ce_lse  # noqa: E402
from workloads import make, workload  # noqa: E402


def main():
    inp = make(workload("llm_ce"))
    A = decode_bf16(inp["A"])
    E = decode_bf16(inp["E"])
    T = A.shape[0]
    lse = np.empty(T, dtype=np.float64)
    step = 256
    for r0 in range(0, T, step):
        rows = np.arange(r0, min(T, r0 + step))
        lse[rows] = ce_lse(A, E, rows)
        print(f"rows {r0}..{rows[-1]}", flush=True)
    np.save(os.path.join(os.path.dirname(os.path.abspath(__file__)), "llm_ce_lse.npy"), lse)


if __name__ == "__main__":
    main()
