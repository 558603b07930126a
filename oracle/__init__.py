"""CPU oracle for the small-M W4A16 NVFP4 GEMV family.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
The arithmetic lives in ``nvfp4_oracle.c`` (plain C, IEEE binary64); this
package is its ctypes front end.
"""
from .oracle import *  # noqa: F401,F403
