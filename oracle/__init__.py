"""CPU oracle for the NVFP4 block-scaled path (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It wraps ``liboracle.so`` (plain C, see
``nvfp4_oracle.c``) with numpy marshalling and shares nothing with the HIP
library.

Parity unpinned: none of the functions here is without a pin; see
``tests/test_oracle_*.py`` for what fixes each one.
"""
from .oracle import *  # noqa: F401,F403
