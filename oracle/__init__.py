"""fp64 CPU oracle of the SPIN decode step -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the HIP library and its Python binding never do.
"""
from . import spin_oracle  # noqa: F401
