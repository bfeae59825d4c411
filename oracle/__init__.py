"""CPU oracle for the fused large-vocabulary classifier-head losses.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or call anything in this package; the
product path never does, and it shares no code with the HIP kernels.

Everything is plain NumPy in float64 over the exact values of the bf16/fp8
input bytes. Where the method reaches a result that has a plain definition
(the BCE and CE losses and their gradients), the oracle writes that definition
out: it materializes the logits X = A E^T and evaluates the loss elementwise.

Modules:
  formats    bf16 / OCP FP8 E4M3FN decoding and FP8 encoding (own code)
  targets    canonical positive sets, item-major pairs
  head_loss  BCE and CE loss/gradients (full and sampled), fused FP8 SGD

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, the dense+sparse identity, torch's library BCE/CE with
autograd, finite differences and invariants (listed in each test).
"""
from . import formats, targets, head_loss  # noqa: F401
