"""CPU oracle for the RDKV hot path -- test infrastructure only.

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this package.  The HIP library never calls it and shares
no code with it.
"""
from .rdkv_oracle import *  # noqa: F401,F403
