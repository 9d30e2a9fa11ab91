"""CPU oracle for the EAGLE-3 draft-and-verify hot path.

TEST INFRASTRUCTURE ONLY.  Plain, slow NumPy (float64) restatement of what the
path computes, used by the tests, the smoke check and the CPU-baseline leg of
the benchmark.  The product path never imports it.
"""
from .eagle_oracle import *  # noqa: F401,F403
from .eagle_oracle import __all__  # noqa: F401
