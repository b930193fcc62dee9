"""CPU oracle (test infrastructure only; see dynrad_oracle.py)."""
from .dynrad_oracle import *  # noqa: F401,F403
