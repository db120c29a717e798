"""CPU oracle (test infrastructure only; see esg_oracle's header)."""
from .esg_oracle import *  # noqa: F401,F403
