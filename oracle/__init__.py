"""CPU oracle (test infrastructure only; see oracle/verify.py).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The HIP library never does, and the oracle uses none of its code.
"""
from .verify import *  # noqa: F401,F403
from .verify import __all__  # noqa: F401
