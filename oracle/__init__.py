"""CPU oracle (test infrastructure only; see fp4_oracle's header)."""
from . import fp4_oracle  # noqa: F401
from .fp4_oracle import *  # noqa: F401,F403
