"""CPU oracle (test infrastructure only; see flashprefill_oracle)."""
from .flashprefill_oracle import *  # noqa: F401,F403
