"""CPU oracle for the OPQ W4A16 hot path.

Test infrastructure only: the test suite, the smoke check and the CPU
baseline leg of the benchmark may use this package. The library and its
Python binding never import it.
"""
from .opq_oracle import *  # noqa: F401,F403
