"""CPU oracle of the linear cross-entropy (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does.
"""
from . import lce_oracle  # noqa: F401
