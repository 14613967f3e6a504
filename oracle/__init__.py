"""CPU oracle for the CSA hot path (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. The HIP library and its Python binding never do.
"""
from .csa_oracle import *  # noqa: F401,F403
