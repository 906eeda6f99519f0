"""fp64 CPU oracle (test infrastructure only; see sla_oracle.py)."""
from .sla_oracle import *  # noqa: F401,F403
from . import sla_oracle  # noqa: F401
