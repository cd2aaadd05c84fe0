"""CPU oracle (float64 NumPy) for the RBS prefill-attention hot path.

Test infrastructure only: imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product package.
"""
from . import rbs_oracle  # noqa: F401
