"""CPU oracle (test infrastructure only; see fp8_oracle.py's header)."""
from .fp8_oracle import *  # noqa: F401,F403
from .fp8_oracle import FP8_MAX, BLOCK  # noqa: F401
