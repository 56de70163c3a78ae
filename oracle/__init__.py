"""CPU oracle (test infrastructure only; see hisa_oracle.py's header)."""
from .hisa_oracle import *  # noqa: F401,F403
