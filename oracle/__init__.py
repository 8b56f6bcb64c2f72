"""CPU oracle for the Gated DeltaNet token mixer (plain fp64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from . import gdn_oracle, checkers  # noqa: F401
