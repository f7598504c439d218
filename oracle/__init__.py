"""CPU oracle of the CSA2 hot path (test infrastructure only; see csa2_oracle)."""
from .csa2_oracle import *  # noqa: F401,F403
from . import csa2_oracle  # noqa: F401
