"""CPU oracle (test infrastructure only; see ssa_oracle's module docstring)."""
from .ssa_oracle import *  # noqa: F401,F403
