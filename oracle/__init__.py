"""fp64 CPU oracle for the DSA/SWA hot path -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product path never does.
"""
from .dsa_oracle import *  # noqa: F401,F403
from . import cache_append  # noqa: F401
