"""fp64 CPU oracle (test infrastructure only; see flux_oracle.py's header)."""
from .flux_oracle import *  # noqa: F401,F403
from . import flux_oracle  # noqa: F401
