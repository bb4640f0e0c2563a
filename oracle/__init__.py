"""CPU float64 oracle -- test infrastructure only (tests, smoke, cpu_baseline).

The product library never imports this package.
"""
from . import oracle, step, compare  # noqa: F401
