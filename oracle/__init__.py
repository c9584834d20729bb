"""CPU oracle of the Engram forward: test infrastructure only (see engram_oracle.py)."""
from .engram_oracle import *  # noqa: F401,F403
from . import engram_oracle  # noqa: F401
