"""CPU oracle (test infrastructure only; see qmm_oracle's header)."""
from . import qmm_oracle, brute  # noqa: F401
