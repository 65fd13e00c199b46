"""CPU fp64 oracle for CSA / HCA attention -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does."""
from .csa_oracle import *  # noqa: F401,F403
