"""CPU oracle for exact attention (fp64, numpy).

TEST INFRASTRUCTURE. Nothing in the product path imports this package: only
the tests, the package smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library (no kernels, headers, helpers or
tables), and imports nothing from it.

  attention_ref  -- three-step S -> P -> O forward, backward, decode
  online_model   -- the per-row online-softmax recurrence and partial merge
  philox         -- Philox counter-based random numbers (the dropout mask)
"""
from . import attention_ref, online_model, philox  # noqa: F401
