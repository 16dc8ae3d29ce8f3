"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .dsa_oracle import *  # noqa: F401,F403
