"""fp64 CPU oracle of the MC-Sparse hot path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
bench's CPU-baseline leg, never by the product path.
"""
from .mcs_oracle import *  # noqa: F401,F403
