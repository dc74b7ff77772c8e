"""CPU oracle (test infrastructure only; see oracle.oracle)."""
from . import oracle  # noqa: F401
