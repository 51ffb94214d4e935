"""CPU oracle package (test infrastructure only; see hisa_oracle)."""
from .hisa_oracle import *  # noqa: F401,F403
