"""CPU oracle for the MixQ-style mixed-precision linear layer.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
"""
from .mixq_oracle import *  # noqa: F401,F403
