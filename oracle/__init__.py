"""CPU oracle of the DFlash 2 proposer hot path (test infrastructure only)."""
from .dflash2_oracle import *  # noqa: F401,F403
