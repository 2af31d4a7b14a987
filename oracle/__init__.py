"""fp64 CPU oracle for the CONF-KV decode step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""
from .confk_oracle import *  # noqa: F401,F403
