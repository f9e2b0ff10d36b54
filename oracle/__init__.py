"""fp64 CPU oracle of the block-sparse video attention path (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it, and it shares no code
with the HIP path.
"""
from .svsa_oracle import *  # noqa: F401,F403
from .svsa_oracle import __all__  # noqa: F401
