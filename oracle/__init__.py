"""CPU oracle (float64, numpy) for the CSA/HCA hybrid compressed attention path.

Test infrastructure: importable only by the tests, the smoke check and the benchmark's
CPU-baseline leg.  It shares no code with the HIP library.
"""
from .hcsa_oracle import *  # noqa: F401,F403
