"""CPU oracle (test infrastructure only; never used by the product path)."""
from .hla_oracle import *  # noqa: F401,F403
