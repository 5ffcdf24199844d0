"""CPU oracle (test infrastructure only; see oracle/verify.py, oracle/ngram.py and oracle/adaptive.py).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The HIP library never does, and the oracle uses none of its code.
"""
from .verify import *  # noqa: F401,F403
from .verify import __all__ as _verify_all
from .ngram import *  # noqa: F401,F403
from .ngram import __all__ as _ngram_all
from .adaptive import *  # noqa: F401,F403
from .adaptive import __all__ as _adaptive_all

__all__ = list(_verify_all) + list(_ngram_all) + list(_adaptive_all)
