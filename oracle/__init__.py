"""fp64 CPU oracle for GroupQueryAttention over a shared-buffer KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its Python binding.
It shares no code with the HIP path.

  gqa_oracle  vectorised numpy fp64 definition of every step
  brute       scalar-loop twin used to pin gqa_oracle on tiny inputs

Parity status of each function: every function is pinned by the tests in
tests/test_oracle_pins.py (brute force, a library routine on a special case,
closed forms and invariants); none is "parity unpinned".
"""
from . import gqa_oracle, brute  # noqa: F401
